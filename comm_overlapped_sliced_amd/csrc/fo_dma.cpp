// DMA transfer layer of libflashovl: emulated point-to-point transfers on the SDMA engines.
//
// The FlashOverlap page (gist.science paper 2604.24013, technical summary section 2) splits the
// collectives into point-to-point transfers that run while the GEMM computes; section 3 credits
// the method with relaxing the step-wise synchronisation of the collective. On one GPU a transfer
// is a copy from a "peer" buffer, and what matters is that it neither takes compute units from
// the GEMM nor needs one to be scheduled: the GEMM may hold every CU while it waits for the very
// slice being copied. So each transfer is an SDMA copy issued through the HSA runtime with its
// dependencies given as signals that the engine itself polls (the start of the call, and for
// Flash-RS in lockstep the release of a GEMM step), and its completion is a signal whose value
// the kernels poll. One engine stands for one link: transfers on the same link run one after
// the other in issue order, transfers on different links run concurrently.
//
// The HSA entry points are those of the HSA runtime instance that HIP itself runs on.
#include <dlfcn.h>
#include <link.h>
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include <algorithm>
#include <bitset>
#include <chrono>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <thread>
#include <type_traits>
#include <vector>

#include "fo_internal.h"

namespace fo {
namespace dma {
namespace {

struct Hsa {
  decltype(&hsa_amd_pointer_info) pointer_info = nullptr;
  decltype(&hsa_amd_memory_copy_engine_status) engine_status = nullptr;
  decltype(&hsa_amd_signal_create) signal_create = nullptr;
  decltype(&hsa_amd_signal_value_pointer) value_pointer = nullptr;
  decltype(&hsa_signal_store_screlease) store = nullptr;
  decltype(&hsa_signal_load_scacquire) load = nullptr;
  decltype(&hsa_amd_memory_async_copy_on_engine) copy = nullptr;
};

Hsa g_hsa;
bool g_hsa_ok = false;
std::string g_hsa_err;

int collect_hsa(struct dl_phdr_info* info, size_t, void* data) {
  if (info->dlpi_name && strstr(info->dlpi_name, "libhsa-runtime64.so"))
    static_cast<std::vector<std::string>*>(data)->push_back(info->dlpi_name);
  return 0;
}

bool table_of(void* h, Hsa* t, std::string* err) {
  bool ok = true;
  auto get = [&](auto& fn, const char* name) {
    fn = reinterpret_cast<std::remove_reference_t<decltype(fn)>>(dlsym(h, name));
    if (!fn) {
      ok = false;
      *err = std::string("the HSA runtime lacks ") + name;
    }
  };
  get(t->pointer_info, "hsa_amd_pointer_info");
  get(t->engine_status, "hsa_amd_memory_copy_engine_status");
  get(t->signal_create, "hsa_amd_signal_create");
  get(t->value_pointer, "hsa_amd_signal_value_pointer");
  get(t->store, "hsa_signal_store_screlease");
  get(t->load, "hsa_signal_load_scacquire");
  get(t->copy, "hsa_amd_memory_async_copy_on_engine");
  return ok;
}

// Picks the HSA runtime HIP runs on. A process can hold more than one copy of the runtime (a
// profiler's tool library brings its own), and only the instance HIP initialized knows HIP's
// allocations: the runtime chosen is the one that recognizes `dev_ptr`, a hipMalloc'ed buffer.
void resolve_hsa(const void* dev_ptr) {
  std::vector<std::string> libs;
  dl_iterate_phdr(collect_hsa, &libs);
  g_hsa_err = "no HSA runtime in the process knows the library's device allocation";
  for (const std::string& lib : libs) {
    void* h = dlopen(lib.c_str(), RTLD_NOW | RTLD_NOLOAD);
    if (!h) continue;
    Hsa t;
    std::string e;
    if (!table_of(h, &t, &e)) {
      g_hsa_err = e + " (" + lib + ")";
      continue;
    }
    hsa_amd_pointer_info_t info;
    memset(&info, 0, sizeof info);
    info.size = sizeof info;
    if (t.pointer_info(dev_ptr, &info, nullptr, nullptr, nullptr) == HSA_STATUS_SUCCESS &&
        info.type == HSA_EXT_POINTER_TYPE_HSA) {
      g_hsa = t;
      g_hsa_ok = true;
      return;
    }
  }
}

constexpr int kSignals = FO_MAX_P * kMaxGroups;  // per kind and slot: [slice or position][group]

struct Slot {
  hsa_signal_t start{}, rel[kSignals]{}, comp[kSignals]{};
  int64_t* start_v = nullptr;
  int64_t** tab = nullptr;  // device: comp values [kSignals], then rel values [kSignals]
  hipEvent_t ev = nullptr;  // recorded after the call's last kernel that reads the signals
  bool pending = false;     // used by a call that may not be complete yet
  std::bitset<kSignals> issued;  // completion signals a copy will decrement
  uint32_t started = 0;          // engines that already hold a copy of the call waiting on start
  uint8_t turn[32] = {};         // per engine pair: copies the call has issued on it
};

struct Dev {
  bool ready = false;
  hsa_agent_t agent{};
  int n_eng = 0;
  uint32_t eng[32] = {};
  int n_pairs = 0;  // eng[i] and eng[i + n_pairs] form a pair (engines 2k and 2k+1), i < n_pairs
  Slot slot[kSlots];
  int next = 0;
};

constexpr int kMaxDevices = 64;
Dev g_dev[kMaxDevices];

constexpr size_t kWarmBytes = 65536;
constexpr size_t kSplitMin = 65536;  // a transfer is split across a pair only if each half is this big

const char* hsa_msg(hsa_status_t s) {
  switch (s) {
    case HSA_STATUS_SUCCESS: return "success";
    case HSA_STATUS_ERROR_INVALID_ARGUMENT: return "invalid argument";
    case HSA_STATUS_ERROR_INVALID_AGENT: return "invalid agent";
    case HSA_STATUS_ERROR_INVALID_SIGNAL: return "invalid signal";
    case HSA_STATUS_ERROR_OUT_OF_RESOURCES: return "out of resources";
    case HSA_STATUS_ERROR_NOT_INITIALIZED: return "runtime not initialized";
    default: return "error";
  }
}

bool fail(std::string* err, const char* what, hsa_status_t s) {
  char buf[256];
  snprintf(buf, sizeof buf, "%s failed: %s (0x%x)", what, hsa_msg(s), (unsigned)s);
  *err = buf;
  return false;
}

bool new_signal(hsa_signal_t* sig, int64_t** value, std::string* err) {
  hsa_status_t s = g_hsa.signal_create(1, 0, nullptr, HSA_AMD_SIGNAL_AMD_GPU_ONLY, sig);
  if (s != HSA_STATUS_SUCCESS) return fail(err, "hsa_amd_signal_create", s);
  volatile hsa_signal_value_t* v = nullptr;
  s = g_hsa.value_pointer(*sig, &v);
  if (s != HSA_STATUS_SUCCESS) return fail(err, "hsa_amd_signal_value_pointer", s);
  *value = (int64_t*)v;
  return true;
}

// Host wait (bounded) until the completion signal of every issued slice has dropped to zero.
bool wait_landed(const Slot& sl, uint32_t timeout_ms, std::string* err, bool* timed_out = nullptr) {
  const auto t0 = std::chrono::steady_clock::now();
  for (int i = 0; i < kSignals; ++i) {
    if (!sl.issued[i]) continue;
    int spins = 0;
    for (;;) {
      const int64_t v = g_hsa.load(sl.comp[i]);
      if (v < 0) {
        *err = "a DMA transfer reported failure";
        return false;
      }
      if (v == 0) break;
      if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(timeout_ms)) {
        *err = "a DMA transfer did not complete within its bound";
        if (timed_out) *timed_out = true;
        return false;
      }
      if (++spins > 64) std::this_thread::sleep_for(std::chrono::microseconds(50));
    }
  }
  return true;
}

}  // namespace

bool init(int dev, void* scratch, std::string* err) {
  if (dev < 0 || dev >= kMaxDevices) {
    *err = "device index beyond the DMA layer's limit";
    return false;
  }
  Dev& d = g_dev[dev];
  if (d.ready) return true;
  {
    static std::mutex m;  // devices initialize under their own locks
    std::lock_guard<std::mutex> lk(m);
    if (!g_hsa_ok) resolve_hsa(scratch);
    if (!g_hsa_ok) {
      *err = g_hsa_err;
      return false;
    }
  }
  // the runtime is up: HIP initialized it before it allocated `scratch`
  hsa_amd_pointer_info_t info;
  memset(&info, 0, sizeof info);
  info.size = sizeof info;
  hsa_status_t s = g_hsa.pointer_info(scratch, &info, nullptr, nullptr, nullptr);
  if (s != HSA_STATUS_SUCCESS) return fail(err, "hsa_amd_pointer_info", s);
  if (info.type != HSA_EXT_POINTER_TYPE_HSA) {
    *err = "the library's scratch buffer is not device memory of the HSA runtime";
    return false;
  }
  d.agent = info.agentOwner;
  // Engines for device-to-device copies. Runtimes that cannot report them for a copy within one
  // device get ids 2..15 tried (0 and 1 are left to HIP's own copies, as the runtimes that do
  // report them leave them out); an id whose first copy the runtime refuses is dropped.
  uint32_t mask = 0;
  s = g_hsa.engine_status(d.agent, d.agent, &mask);
  if (s != HSA_STATUS_SUCCESS || mask == 0) mask = 0xfffcu;
  d.n_eng = 0;
  for (int i = 0; i < 32; ++i)
    if (mask & (1u << i)) d.eng[d.n_eng++] = 1u << i;
  std::vector<int64_t*> values(2 * kSignals);
  for (Slot& sl : d.slot) {
    if (!new_signal(&sl.start, &sl.start_v, err)) return false;
    for (int i = 0; i < kSignals; ++i) {
      if (!new_signal(&sl.comp[i], &values[i], err)) return false;
      if (!new_signal(&sl.rel[i], &values[kSignals + i], err)) return false;
    }
    if (hipMalloc((void**)&sl.tab, values.size() * sizeof(int64_t*)) != hipSuccess ||
        hipMemcpy(sl.tab, values.data(), values.size() * sizeof(int64_t*),
                  hipMemcpyHostToDevice) != hipSuccess) {
      *err = "cannot place the signal tables in device memory";
      return false;
    }
    if (hipEventCreateWithFlags(&sl.ev, hipEventDisableTiming) != hipSuccess) {
      *err = "hipEventCreateWithFlags failed";
      return false;
    }
  }
  // one small copy per engine, one engine at a time
  Slot& w = d.slot[0];
  uint8_t* src = (uint8_t*)scratch;
  int kept = 0;
  for (int e = 0; e < d.n_eng; ++e) {
    g_hsa.store(w.comp[0], 1);
    s = g_hsa.copy(src + kWarmBytes, d.agent, src, d.agent, kWarmBytes, 0, nullptr, w.comp[0],
                   (hsa_amd_sdma_engine_id_t)d.eng[e], true);
    if (s != HSA_STATUS_SUCCESS) continue;
    w.issued.reset();
    w.issued.set(0);
    if (!wait_landed(w, 10000, err)) return false;
    d.eng[kept++] = d.eng[e];
  }
  d.n_eng = kept;
  if (kept == 0) {
    *err = "no SDMA engine accepts device-to-device copies on this device";
    return false;
  }
  // Engines 2k and 2k+1 share their bandwidth: measured on MI355X, seven concurrent 16 MiB copies
  // on engines 2..8 run at ~46 GB/s each, on engines 2, 4, ..., 14 at ~58 GB/s each (one engine
  // alone: ~59 GB/s). Links take one engine of each pair before the second of any pair.
  std::stable_partition(d.eng, d.eng + d.n_eng, [](uint32_t bit) {
    return (__builtin_ctz(bit) & 1) == 0;
  });
  // engine pairs for links of two engines: the even engine i and its odd partner i + n_pairs,
  // when every even engine has its partner in place
  const int half = d.n_eng / 2;
  bool paired = d.n_eng % 2 == 0 && half > 0;
  for (int i = 0; paired && i < half; ++i) paired = d.eng[i + half] == (d.eng[i] << 1);
  d.n_pairs = paired ? half : 0;
  w.issued.reset();
  d.ready = true;
  return true;
}

int n_engines(int dev) { return (dev >= 0 && dev < kMaxDevices) ? g_dev[dev].n_eng : 0; }

bool begin(int dev, int P, int groups, Call* call, std::string* err) {
  Dev& d = g_dev[dev];
  if (!d.ready) {
    *err = "DMA layer not initialized";
    return false;
  }
  if (P < 1 || P > FO_MAX_P || groups < 1 || groups > kMaxGroups) {
    *err = "slice or group count beyond the DMA layer's signal slots";
    return false;
  }
  const int k = d.next;
  Slot& sl = d.slot[k];
  if (sl.pending) {
    if (hipEventSynchronize(sl.ev) != hipSuccess) {
      *err = "hipEventSynchronize on a previous call failed";
      return false;
    }
    if (!wait_landed(sl, 30000, err)) return false;
    sl.pending = false;
  }
  g_hsa.store(sl.start, 1);
  for (int i = 0; i < P; ++i)
    for (int g = 0; g < groups; ++g) {
      g_hsa.store(sl.rel[i * kMaxGroups + g], 1);
      g_hsa.store(sl.comp[i * kMaxGroups + g], 1);
    }
  sl.issued.reset();
  sl.started = 0;
  memset(sl.turn, 0, sizeof sl.turn);
  sl.pending = true;
  d.next = (k + 1) % kSlots;
  call->slot = k;
  call->start = sl.start_v;
  call->comp_tab = sl.tab;
  call->rel_tab = sl.tab + kSignals;
  return true;
}

bool copy(int dev, const Call& call, int link, int slice, int group, int rel_pos, void* dst,
          const void* src, size_t bytes, std::string* err) {
  Dev& d = g_dev[dev];
  Slot& sl = d.slot[call.slot];
  const int ci = slice * kMaxGroups + group;
  if (bytes == 0) {
    g_hsa.store(sl.comp[ci], 0);
    return true;
  }
  // An engine runs its copies one after the other in issue order, so only the call's first copy
  // on an engine waits for the start signal; a copy gated on a release signal needs no start
  // signal at all (the kernel stores the release after it has started).
  // the engines of this copy: one; or the pair's next in turn; or (split) both halves of the
  // transfer, one on each engine of the pair, counted down on the same completion signal
  int ei[2] = {(link % d.n_eng + d.n_eng) % d.n_eng, -1};
  size_t part[2] = {bytes, 0};
  if (call.pairs && d.n_pairs > 0) {
    const int pr = (link % d.n_pairs + d.n_pairs) % d.n_pairs;
    if (call.split && bytes >= 2 * kSplitMin) {
      ei[0] = pr;
      ei[1] = pr + d.n_pairs;
      part[0] = (bytes / 2 + 255) / 256 * 256;  // the first half ends on a 256-byte boundary
      part[1] = bytes - part[0];
      g_hsa.store(sl.comp[ci], 2);
    } else {
      ei[0] = pr + (sl.turn[pr]++ & 1) * d.n_pairs;
    }
  }
  size_t off = 0;
  for (int k = 0; k < 2 && ei[k] >= 0; ++k) {
    const uint32_t eng = d.eng[ei[k]];
    hsa_signal_t deps[1];
    uint32_t n = 0;
    if (rel_pos >= 0) {
      deps[n++] = sl.rel[rel_pos * kMaxGroups + group];
    } else if (!(sl.started & (1u << ei[k]))) {
      deps[n++] = sl.start;
      sl.started |= 1u << ei[k];
    }
    // (the runtime rejects a dependency array with a count of zero: pass none then)
    const hsa_status_t s =
        g_hsa.copy((uint8_t*)dst + off, d.agent, (const uint8_t*)src + off, d.agent, part[k], n,
                   n ? deps : nullptr, sl.comp[ci], (hsa_amd_sdma_engine_id_t)eng, true);
    if (s != HSA_STATUS_SUCCESS) {
      // the kernel must not wait for a copy that was never issued: report it as failed (a half
      // already issued still counts the signal down, so it stays negative)
      g_hsa.store(sl.comp[ci], -(int64_t)16);
      sl.issued.set(ci);
      return fail(err, "hsa_amd_memory_async_copy_on_engine", s);
    }
    off += part[k];
  }
  sl.issued.set(ci);
  return true;
}

bool end(int dev, const Call& call, hipStream_t stream, std::string* err, hipEvent_t* ev) {
  if (hipEventRecord(g_dev[dev].slot[call.slot].ev, stream) != hipSuccess) {
    *err = "hipEventRecord failed";
    return false;
  }
  if (ev) *ev = g_dev[dev].slot[call.slot].ev;
  return true;
}

bool drain(int dev, uint32_t timeout_ms, std::string* err, bool* timed_out) {
  *timed_out = false;
  if (dev < 0 || dev >= kMaxDevices) return true;
  Dev& d = g_dev[dev];
  if (!d.ready) return true;
  for (Slot& sl : d.slot) {
    if (!sl.pending) continue;
    if (hipEventSynchronize(sl.ev) != hipSuccess) {
      *err = "hipEventSynchronize on a previous call failed";
      return false;
    }
    if (!wait_landed(sl, timeout_ms, err, timed_out)) return false;
    sl.pending = false;
    sl.issued.reset();
  }
  return true;
}

}  // namespace dma
}  // namespace fo
