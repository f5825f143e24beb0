// pa_decode_noalloc: pa_decode with its workspace in a file-scope device
// array, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array below lives in every device's copy of the library's code object.
// In host code its name is only a host-side stand-in: the device address is
// looked up once per device with hipGetSymbolAddress (on the first call made
// with that device current) and only that address is passed to kernels.
// Every call on a device shares the device's array, so calls that overlap on
// one device (on different streams, or from several host threads) race. The
// decode kernels need nothing cleared: each call writes every record and
// partial it later reads.
#include <mutex>

#include "api_internal.h"
#include "device.h"
#include "status.h"

namespace pa {
namespace {

// 32 MiB: the default launch (8 wavefronts per compute unit) of the largest
// unit built (8 query heads of head_dim 128) on 256 compute units needs
// 16.6 MiB.
constexpr size_t kScratchBytes = size_t(32) << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];        // device address of `scratch` on each device
hipError_t g_lookup[kMaxDevices];    // result of the lookup on each device

// Device address of this device's `scratch`, looked up on first use.
pa_status scratch_ptr(void** out, const char* who) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, "%s: device %d beyond the %d supported", who, dev, kMaxDevices);
  std::call_once(g_once[dev], [dev]() {
    void* p = nullptr;
    g_lookup[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_lookup[dev] == hipSuccess ? p : nullptr;
  });
  if (g_lookup[dev] != hipSuccess || !g_scratch[dev])
    return fail(PA_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array on device %d: %s", who,
                dev, hipGetErrorString(g_lookup[dev]));
  *out = g_scratch[dev];
  return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" {

size_t pa_decode_noalloc_scratch_bytes(void) { return pa::kScratchBytes; }

pa_status pa_decode_noalloc(void* out, const void* q, const pa_pool* pool,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                            float scale, int32_t num_workers, void* stream) {
  pa::clear_error();
  const char* who = "pa_decode_noalloc";
  const pa::DecodeCall c{out, q, pool, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                         num_q_heads, scale, num_workers};
  size_t need = 0;
  if (pa_status s = pa::decode_check(c, who, &need)) return s;
  if (num_seqs == 0) return PA_OK;
  if (need > pa::kScratchBytes)
    return pa::fail(PA_ERR_WORKSPACE, "%s: this call needs %zu bytes of scratch; the static "
                    "array holds %zu (fewer num_workers need less)", who, need, pa::kScratchBytes);
  void* ws = nullptr;
  if (pa_status s = pa::scratch_ptr(&ws, who)) return s;
  return pa::decode_launch(c, ws, stream, who);
}

}  // extern "C"
