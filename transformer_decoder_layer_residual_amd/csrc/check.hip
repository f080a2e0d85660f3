// check.hip -- validation of the index inputs of the paged-cache calls.
//
// The ReshapeAndCache / PagedAttention inputs named on the ATB KV-cache page
// (hwcomputing.csdn.net, section "KV cache memory bottleneck") are device
// arrays: block_table, the token positions, the token -> sequence map,
// contextLens, and for packed prefill the cumulative sequence lengths.  The
// compute kernels never fault on a bad entry (they clamp or drop it) but then
// give wrong numbers; this kernel reads the same arrays and reports every
// violated precondition as a bit of one device word, so a debug caller can
// check a call's inputs without a host round trip per array.
//
// One workgroup walks every array (they are at most a few hundred KB) and
// writes the OR of the violation bits with a single plain store, so the word
// needs no clearing before the call.
#include "../../include/dl_layer.h"
#include "dl_internal.hpp"

namespace dl {

constexpr int kCheckThreads = 1024;

__global__ void __launch_bounds__(kCheckThreads)
check_indices_kernel(const int32_t* __restrict__ bt, int B, int max_blocks, int num_blocks, int BS,
                     const int32_t* __restrict__ pos, const int32_t* __restrict__ seq, int T,
                     const int32_t* __restrict__ ctx, int max_ctx,
                     const int32_t* __restrict__ cu, int max_seqlen, int32_t* __restrict__ word) {
  __shared__ int flags;
  if (threadIdx.x == 0) flags = 0;
  __syncthreads();
  int f = 0;
  const int64_t cap = (int64_t)max_blocks * BS;
  // tokens: sequence id, position, and the table entry the cache write uses
  for (int t = threadIdx.x; t < T; t += kCheckThreads) {
    const int s = seq ? seq[t] : t;
    const int p = pos ? pos[t] : -1;
    bool s_ok = s >= 0 && s < B;
    if (!s_ok) f |= DL_CHECK_BIT_SEQ;
    bool p_ok = true;
    if (pos) {
      p_ok = p >= 0 && p < cap;
      if (!p_ok) f |= DL_CHECK_BIT_POSITION;
    }
    if (pos && bt && s_ok && p_ok) {
      const int blk = bt[(int64_t)s * max_blocks + p / BS];
      if (blk < 0 || blk >= num_blocks) f |= DL_CHECK_BIT_BLOCK;
    }
  }
  // sequences: context length, and every table entry attention reads
  if (ctx) {
    for (int b = threadIdx.x; b < B; b += kCheckThreads) {
      const int c = ctx[b];
      if (c < 1 || c > max_ctx || c > cap) {
        f |= DL_CHECK_BIT_CONTEXT;
        continue;
      }
      if (bt) {
        const int nb = (c + BS - 1) / BS;
        for (int j = 0; j < nb; ++j) {
          const int blk = bt[(int64_t)b * max_blocks + j];
          if (blk < 0 || blk >= num_blocks) f |= DL_CHECK_BIT_BLOCK;
        }
      }
    }
  }
  // packed sequences: cu[0] = 0, nondecreasing, cu[B] = T, lengths <= max_seqlen
  if (cu) {
    for (int b = threadIdx.x; b <= B; b += kCheckThreads) {
      const int v = cu[b];
      if (b == 0 && v != 0) f |= DL_CHECK_BIT_CU;
      if (b == B && v != T) f |= DL_CHECK_BIT_CU;
      if (b > 0) {
        const int len = v - cu[b - 1];
        if (len < 0 || len > max_seqlen) f |= DL_CHECK_BIT_CU;
      }
    }
  }
  if (f) atomicOr(&flags, f);
  __syncthreads();
  if (threadIdx.x == 0) *word = flags;
}

hipError_t check_indices(const int32_t* bt, int B, int max_blocks, int num_blocks, int BS,
                         const int32_t* pos, const int32_t* seq, int T, const int32_t* ctx,
                         int max_ctx, const int32_t* cu, int max_seqlen, int32_t* word,
                         hipStream_t st) {
  hipLaunchKernelGGL(check_indices_kernel, dim3(1), dim3(kCheckThreads), 0, st, bt, B, max_blocks,
                     num_blocks, BS, pos, seq, T, ctx, max_ctx, cu, max_seqlen, word);
  return hipGetLastError();
}

}  // namespace dl
