// Glue kernels around the parallel-draft step: the autoregressive baseline's
// per-pass row builder, and the next round's verified batch.
#include "common.h"

namespace pe {
namespace {

// One autoregressive drafting pass k >= 1 ("P-EAGLE: Parallel Speculative
// Decoding in vLLM", Solving the Autoregressive Drafting Bottleneck: the
// sequential baseline drafts one token per forward pass).  Block i: store
// token k-1 of sequence i, then build the single draft row of pass k: the
// token just drafted at position base_i + k (base_i = position of the
// sequence's bonus row), its cache slot, and as hidden input the drafter's
// own final residual of the row that produced the token, rounded to the
// model dtype.
template <typename T>
__global__ __launch_bounds__(256) void ar_step_kernel(ArStepArgs a) {
  const int i = blockIdx.x;
  const int tok = a.prev_tokens[i];
  if (threadIdx.x == 0) {
    a.draft_tokens[static_cast<int64_t>(i) * a.K + a.k - 1] = tok;
    if (!a.last) {
      const int p = a.base_kv_lens[i] - 1 + a.k;
      a.ids[i] = tok;
      a.pos[i] = p;
      a.slot[i] = static_cast<int64_t>(a.block_table[static_cast<int64_t>(i) * a.max_blocks + p / 16]) * 16 + p % 16;
      a.rejected[i] = 0;
      a.cu_draft[i] = i;
      if (i == a.c - 1) a.cu_draft[a.c] = a.c;
      a.kv_lens[i] = p + 1;
      a.sample_idx[i] = i;
    }
  }
  if (a.last) return;
  const int row = a.prev_sample_idx ? a.prev_sample_idx[i] : i;
  const float* x = a.x + static_cast<int64_t>(row) * a.H;
  T* h = static_cast<T*>(a.hidden) + static_cast<int64_t>(i) * a.H;
  for (int e = threadIdx.x; e < a.H; e += blockDim.x) h[e] = Elem<T>::from_f32(x[e]);
}

// Next round's verified batch: the target model verified, for sequence i, the
// K + 1 rows [bonus, d_0 .. d_{K-1}] at positions base_i + 1 .. base_i + K + 1
// (base_i = kv_lens[i] - K, the position of this round's bonus row), accepted
// acc_next[i] of the drafts and supplied bonus_next[i].
__global__ __launch_bounds__(256) void next_batch_kernel(int c, int K, const int32_t* kv_lens,
                                                         const int32_t* bonus, const int32_t* drafts,
                                                         const int32_t* acc_next, const int32_t* bonus_next,
                                                         int32_t* query_lens, int32_t* target_ids,
                                                         int32_t* target_pos, int32_t* num_accepted,
                                                         int32_t* bonus_ids) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= c) return;
  const int base = kv_lens[i] - K;
  const int64_t r0 = static_cast<int64_t>(i) * (K + 1);
  target_ids[r0] = bonus[i];
  target_pos[r0] = base + 1;
  for (int j = 0; j < K; ++j) {
    target_ids[r0 + 1 + j] = drafts[static_cast<int64_t>(i) * K + j];
    target_pos[r0 + 1 + j] = base + 2 + j;
  }
  query_lens[i] = K + 1;
  num_accepted[i] = acc_next[i];
  bonus_ids[i] = bonus_next[i];
}

}  // namespace

hipError_t launch_ar_step(const ArStepArgs& a, hipStream_t s) {
  if (a.dtype == DType::F32)
    hipLaunchKernelGGL(ar_step_kernel<float>, dim3(a.c), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(ar_step_kernel<bf16_t>, dim3(a.c), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_next_batch(int c, int K, const int32_t* kv_lens, const int32_t* bonus, const int32_t* drafts,
                             const int32_t* acc_next, const int32_t* bonus_next, int32_t* query_lens,
                             int32_t* target_ids, int32_t* target_pos, int32_t* num_accepted, int32_t* bonus_ids,
                             hipStream_t s) {
  hipLaunchKernelGGL(next_batch_kernel, dim3((c + 255) / 256), dim3(256), 0, s, c, K, kv_lens, bonus, drafts,
                     acc_next, bonus_next, query_lens, target_ids, target_pos, num_accepted, bonus_ids);
  return hipGetLastError();
}

}  // namespace pe
