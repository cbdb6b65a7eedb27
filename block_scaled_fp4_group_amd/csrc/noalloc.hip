// Router + permutation for callers that cannot allocate: the hand-off counter
// and the permutation's count table live in one file-scope device array
// (`scratch`), so the call takes only the caller's inputs and outputs.
//
// Each GPU holds its own copy of the array for the life of the process.  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in symbol): the device address is looked up once per device with
// hipGetSymbolAddress and kept in g_scratch[device].  Every call on a GPU
// shares that GPU's array, so calls that overlap on one GPU (different streams
// without ordering between them) race.
#include <mutex>

#include "common.h"

namespace moe {

moe_status launch_route(const float*, const float*, int64_t, const moe_route_params*, int32_t*, float*, hipStream_t);
moe_status launch_permute(const int32_t*, int64_t, int, int, int32_t*, int32_t*, int32_t*, void*, hipStream_t);
bool route_permute_fits(int64_t T, int top_k);
size_t permute_ws_bytes(int64_t R, int E);
moe_status launch_route_permute(const float*, const float*, int64_t, const moe_route_params*, int32_t*, float*, int32_t*,
                                int32_t*, int32_t*, uint32_t*, hipStream_t);

// bytes 0..255: the fused kernel's hand-off counter (zero between calls);
// bytes 256..: the multi-chunk permutation's [chunks, E] count table
constexpr size_t kScratchCounterBytes = 256;
constexpr size_t kScratchTableBytes = (size_t)256 << 10;
__device__ __align__(256) uint8_t scratch[kScratchCounterBytes + kScratchTableBytes];

constexpr int kMaxDevices = 64;
static void* g_scratch[kMaxDevices];
static bool g_cleared[kMaxDevices];
static std::mutex g_scratch_mu;

__global__ void clear_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The device address of this device's scratch array (looked up once per
// device, with that device current); nullptr and an error message on failure.
// The counter is cleared by a fill kernel on `stream` before its first use.
static uint8_t* device_scratch(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("moe_route_permute_noalloc: no current HIP device (or device index >= %d)", kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      set_error("moe_route_permute_noalloc: hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                hipGetErrorString(e));
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  if (!g_cleared[dev]) {
    hipLaunchKernelGGL(clear_words, dim3(1), dim3(64), 0, stream, (uint32_t*)g_scratch[dev],
                       (int)(kScratchCounterBytes / 4));
    if (launch_status("moe_route_permute_noalloc(clear)") != MOE_OK) return nullptr;
    g_cleared[dev] = true;
  }
  return (uint8_t*)g_scratch[dev];
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route_permute_noalloc(const float* logits, const float* correction_bias, int64_t T,
                                                const moe_route_params* p, int32_t* topk_ids, float* topk_weights,
                                                int32_t* expert_offsets, int32_t* sorted_slots, int32_t* slot_rows,
                                                hipStream_t stream) {
  set_error("");
  if (!p) {
    set_error("moe_route_permute_noalloc: params is NULL");
    return MOE_ERR_INVALID;
  }
  if (T < 0 || p->num_experts < 2 || p->num_experts > 256 || p->n_group < 1 || p->n_group > 64 ||
      p->num_experts % p->n_group != 0 || p->num_experts / p->n_group < 2 || p->topk_group < 1 ||
      p->topk_group > p->n_group || p->top_k < 1 || p->top_k > 16 ||
      p->top_k > p->topk_group * (p->num_experts / p->n_group)) {
    set_error("moe_route_permute_noalloc: bad T or routing parameters (see moe_route)");
    return MOE_ERR_INVALID;
  }
  if (!expert_offsets) {
    set_error("moe_route_permute_noalloc: expert_offsets is NULL");
    return MOE_ERR_INVALID;
  }
  if (T > 0 && !(logits && topk_ids && topk_weights && sorted_slots && slot_rows)) {
    set_error("moe_route_permute_noalloc: NULL pointer");
    return MOE_ERR_INVALID;
  }
  const int64_t R = T * (int64_t)p->top_k;
  const bool fused = route_permute_fits(T, p->top_k);
  if (!fused && permute_ws_bytes(R, p->num_experts) > kScratchTableBytes) {
    set_error("moe_route_permute_noalloc: %lld slots x %d experts need %zu bytes of count table; the static "
              "scratch holds %zu (at most %lld slots at this expert count)",
              (long long)R, p->num_experts, permute_ws_bytes(R, p->num_experts), kScratchTableBytes,
              (long long)(kScratchTableBytes / (4 * (size_t)p->num_experts)) * 2048);
    return MOE_ERR_UNSUPPORTED;
  }
  uint8_t* s = device_scratch(stream);
  if (!s) return MOE_ERR_HIP;
  if (T == 0) return launch_permute(topk_ids, 0, p->top_k, p->num_experts, expert_offsets, sorted_slots, slot_rows,
                                    s + kScratchCounterBytes, stream);
  if (fused)
    return launch_route_permute(logits, correction_bias, T, p, topk_ids, topk_weights, expert_offsets, sorted_slots,
                                slot_rows, (uint32_t*)s, stream);
  const moe_status rs = launch_route(logits, correction_bias, T, p, topk_ids, topk_weights, stream);
  if (rs != MOE_OK) return rs;
  return launch_permute(topk_ids, T, p->top_k, p->num_experts, expert_offsets, sorted_slots, slot_rows,
                        s + kScratchCounterBytes, stream);
}
