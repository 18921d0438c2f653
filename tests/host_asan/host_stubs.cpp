// Host-only stand-ins for the device side of libidx, so the ABI layer (api.cpp and
// validate.cpp, unchanged) can be built with the host compiler under AddressSanitizer
// and UndefinedBehaviorSanitizer and driven from tests/test_abi_cpu.py without a GPU.
//
// * The two HIP runtime calls the ABI layer makes (current device, its properties)
//   answer "no device" until idx_host_set_device(1) makes device 0 a gfx950 with 256
//   compute units.
// * Every kernel launcher counts its calls and checks what its kernels rely on: the
//   pointers they dereference are non-NULL, the sizes they divide by or loop over are
//   positive, and the launch reached them only with arguments the host checks passed.
//   A failed check counts a violation (idx_host_violations) and returns an error, so a
//   call that would have sent a kernel to a NULL address shows up in the tests.
// Nothing here runs on, or is linked into, the GPU library.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>

#include "../../sparse_attention_indexer_mxfp4_amd/csrc/launch.h"

namespace {

std::atomic<int> g_device_mode{0};
std::atomic<int> g_launches{0};
std::atomic<int> g_violations{0};
char g_static_scratch_tag;

hipError_t verdict(bool ok, const char *what) {
  g_launches.fetch_add(1);
  if (ok) return hipSuccess;
  g_violations.fetch_add(1);
  std::fprintf(stderr, "host stub: %s reached with arguments its kernels cannot use\n", what);
  return hipErrorInvalidValue;
}

}  // namespace

extern "C" {

hipError_t hipGetDevice(int *device) {
  if (!device) return hipErrorInvalidValue;
  if (g_device_mode.load() == 0) return hipErrorNoDevice;
  *device = 0;
  return hipSuccess;
}

hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600 *prop, int device) {
  if (!prop || device != 0 || g_device_mode.load() == 0) return hipErrorInvalidDevice;
  std::memset(prop, 0, sizeof(*prop));
  std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
  prop->multiProcessorCount = 256;
  return hipSuccess;
}

// 0: no device (the default); 1: device 0 is a gfx950 with 256 compute units. The ABI
// layer caches a device's properties on first use, so a device once seen stays gfx950.
void idx_host_set_device(int32_t mode) { g_device_mode.store(mode); }
int32_t idx_host_launches(void) { return g_launches.load(); }
int32_t idx_host_violations(void) { return g_violations.load(); }

}  // extern "C"

namespace idx {

hipError_t launch_mqa_logits(const MqaArgs &a, int num_cus, hipStream_t) {
  // row_start may be NULL (every row starts at key 0)
  bool ok = num_cus > 0 && a.q && a.w && a.row_end && a.logits && a.M > 0 && a.N > 0 && a.H > 0 &&
            a.logits_row_stride >= a.N;
  if (a.paged)
    ok = ok && a.kbase && a.page_size > 0 && a.num_pages > 0 && a.page_stride > 0 && a.key_limit >= 0 &&
         (a.key_limit == 0 || a.block_table);
  else
    ok = ok && a.k && a.k_scale;
  return verdict(ok, "launch_mqa_logits");
}

hipError_t launch_paged_logits(const PagedArgs &a, int num_cus, hipStream_t) {
  bool ok = num_cus > 0 && a.base && a.q && a.w && a.context_lens && a.block_table && a.logits && a.B > 0 &&
            a.next_n > 0 && a.H > 0 && a.width >= 0 && a.page_size > 0 && a.num_pages > 0 && a.page_stride > 0 &&
            a.max_blocks > 0 && (a.fmt == 0 || a.q_scale);
  if (a.block_max) ok = ok && (a.block_size == 16 || a.block_size == 32 || a.block_size == 64);
  if (a.cand) ok = ok && a.n_cand > 0 && a.row_repeat > 0 && a.block_size > 0;
  return verdict(ok, "launch_paged_logits");
}

hipError_t launch_paged_prefill_fp4(const PagedArgs &a, int num_cus, hipStream_t) {
  bool ok = num_cus > 0 && a.base && a.q && a.q_scale && a.w && a.context_lens && a.logits && a.B > 0 && a.H > 0 &&
            a.width > 0 && a.page_size > 0 && a.num_pages > 0 && a.fmt == 1 && (a.max_blocks == 0 || a.block_table);
  return verdict(ok, "launch_paged_prefill_fp4");
}

hipError_t launch_topk(const TopkArgs &a, int num_cus, void *scratch, size_t scratch_bytes, hipStream_t) {
  bool ok = num_cus > 0 && a.logits && a.row_end && a.out && a.rows > 0 && a.width >= 0 && a.k > 0 &&
            a.end_div > 0 && a.out_row_stride >= a.k && a.logits_row_stride >= a.width;
  if (scratch) ok = ok && (scratch_bytes == 0 || scratch_bytes >= topk_scratch_bytes(a.rows) ||
                           a.rows > kCoopMaxRows);
  return verdict(ok, "launch_topk");
}

hipError_t launch_topk_coop(const TopkArgs &, void *, int, hipStream_t) {
  return verdict(false, "launch_topk_coop (only launch_topk may call it)");
}

hipError_t launch_topk_solo(const TopkArgs &, hipStream_t) {
  return verdict(false, "launch_topk_solo (only launch_topk may call it)");
}

void *topk_static_scratch(size_t *bytes) {
  *bytes = topk_scratch_bytes(kCoopMaxRows);
  return &g_static_scratch_tag;
}

hipError_t launch_k_store(const KStoreArgs &a, hipStream_t) {
  bool ok = a.base && a.k && a.slots && a.N > 0 && a.page_size > 0 && a.num_pages > 0 && a.page_stride > 0;
  if (a.norm_weight) ok = ok && a.positions && a.cos_sin && a.max_position > 0 && a.rope_dim > 0;
  return verdict(ok, "launch_k_store");
}

hipError_t launch_q_quant(const QQuantArgs &a, hipStream_t) {
  return verdict(a.q && a.q_out && a.T > 0 && a.H > 0 && (a.fmt == 0 || a.q_scale_out), "launch_q_quant");
}

hipError_t launch_q_rope_quant(const QRopeArgs &a, hipStream_t) {
  return verdict(a.q && a.q_out && a.positions && a.cos_sin && a.weights && a.weights_out && a.T > 0 && a.H > 0 &&
                     a.rope_dim > 0 && a.max_position > 0 && (a.fmt == 0 || a.q_scale_out),
                 "launch_q_rope_quant");
}

hipError_t launch_topk_to_slots(const SlotsArgs &a, hipStream_t) {
  return verdict(a.topk && a.block_table && a.slots && a.indptr && a.rows > 0 && a.k > 0 &&
                     a.page_size > 0 && (a.row_seq || a.next_n > 0),
                 "launch_topk_to_slots");
}

hipError_t launch_candidate_mask(const MaskArgs &a, hipStream_t) {
  return verdict(a.logits && a.row_end && a.cand && a.rows > 0 && a.n_cand > 0 && a.block_size > 0 &&
                     a.row_repeat > 0,
                 "launch_candidate_mask");
}

hipError_t launch_remap_compact_topk(const RemapArgs &a, hipStream_t) {
  return verdict(a.topk && a.cand && a.rows > 0 && a.k > 0 && a.n_cand > 0 && a.block_size > 0 && a.row_repeat > 0,
                 "launch_remap_compact_topk");
}

}  // namespace idx
