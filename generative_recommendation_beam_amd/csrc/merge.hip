// Merge stage (xGR page, section 2.1 xAttention: the stages' local max/sum
// statistics are combined by online softmax). Each part arrives as a
// normalized output o_i and its natural-log lse_i; the combined result is
//   lse = log(sum_i exp(lse_i)),  o = sum_i exp(lse_i - lse) * o_i,
// and a part over no keys (lse_i = -inf) contributes nothing.
// HBM-bound: one thread owns four consecutive floats of one row.
#include "device.h"
#include "kernels.h"

namespace xattn {

namespace {

constexpr int kMergeThreads = 256;

// Rows are never split across blocks (D/4 divides 256), so a block can read
// every lse it needs, wait at a barrier, and only then write lse_out, which
// makes lse_out == lse_a / lse_b safe.
__global__ __launch_bounds__(kMergeThreads) void merge2_kernel(int64_t rows, int D, const float* o_a,
                                                               const float* lse_a, const float* o_b,
                                                               const float* lse_b, float* o_out,
                                                               float* lse_out) {
  const int tpr = D >> 2;
  const int64_t gid = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  const int64_t row = gid / tpr;
  const int c = (int)(gid - row * tpr);
  const bool ok = row < rows;
  float la = neg_inf(), lb = neg_inf();
  if (ok) {
    la = lse_a[row];
    lb = lse_b[row];
  }
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, lse = neg_inf();
  if (m != neg_inf()) {
    wa = exp2_approx((la - m) * kLog2e);  // exp2(-inf) = 0
    wb = exp2_approx((lb - m) * kLog2e);
    const float s = wa + wb;
    lse = m + log2_approx(s) * kLn2;
    const float inv = 1.0f / s;
    wa *= inv;
    wb *= inv;
  }
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  if (ok) {
    const float4 a = reinterpret_cast<const float4*>(o_a + row * D)[c];
    const float4 b = reinterpret_cast<const float4*>(o_b + row * D)[c];
    // a part with weight 0 is skipped so that its contents never matter
    if (wa != 0.f) r = make_float4(wa * a.x, wa * a.y, wa * a.z, wa * a.w);
    if (wb != 0.f) {
      r.x += wb * b.x; r.y += wb * b.y; r.z += wb * b.z; r.w += wb * b.w;
    }
  }
  __syncthreads();
  if (ok) {
    reinterpret_cast<float4*>(o_out + row * D)[c] = r;
    if (lse_out && c == 0) lse_out[row] = lse;
  }
}

__global__ __launch_bounds__(kMergeThreads) void merge_parts_kernel(int64_t rows, int D, int parts,
                                                                    const float* po,
                                                                    const float* plse, float* o,
                                                                    float* lse_out) {
  const int tpr = D >> 2;
  const int64_t gid = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  const int64_t row = gid / tpr;
  const int c = (int)(gid - row * tpr);
  if (row >= rows) return;
  // The loops are unrolled so that several parts' loads are in flight at once
  // (one round trip per few parts instead of one per part); a part with no
  // keys (lse = -inf) is selected away rather than branched around.
  float m = neg_inf();
#pragma unroll 8
  for (int i = 0; i < parts; ++i) m = fmaxf(m, plse[(int64_t)i * rows + row]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lse = neg_inf();
  if (m != neg_inf()) {
    float s = 0.f;
#pragma unroll 4
    for (int i = 0; i < parts; ++i) {
      const float li = plse[(int64_t)i * rows + row];
      const float4 v = reinterpret_cast<const float4*>(po + ((int64_t)i * rows + row) * D)[c];
      const bool on = li != neg_inf();
      const float w = on ? exp2_approx((li - m) * kLog2e) : 0.f;
      acc.x += on ? w * v.x : 0.f;
      acc.y += on ? w * v.y : 0.f;
      acc.z += on ? w * v.z : 0.f;
      acc.w += on ? w * v.w : 0.f;
      s += w;
    }
    const float inv = 1.0f / s;
    acc.x *= inv; acc.y *= inv; acc.z *= inv; acc.w *= inv;
    lse = m + log2_approx(s) * kLn2;
  }
  reinterpret_cast<float4*>(o + row * D)[c] = acc;
  if (lse_out && c == 0) lse_out[row] = lse;
}

}  // namespace

hipError_t launch_merge2(int64_t rows, int D, const float* o_a, const float* lse_a, const float* o_b,
                         const float* lse_b, float* o_out, float* lse_out, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int64_t threads = rows * (D / 4);
  const int64_t blocks = (threads + kMergeThreads - 1) / kMergeThreads;
  hipLaunchKernelGGL(merge2_kernel, dim3((unsigned)blocks), dim3(kMergeThreads), 0, st, rows, D,
                     o_a, lse_a, o_b, lse_b, o_out, lse_out);
  return hipGetLastError();
}

hipError_t launch_merge_parts(int64_t rows, int D, int parts, const float* po, const float* plse,
                              float* o, float* lse, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int64_t threads = rows * (D / 4);
  const int64_t blocks = (threads + kMergeThreads - 1) / kMergeThreads;
  hipLaunchKernelGGL(merge_parts_kernel, dim3((unsigned)blocks), dim3(kMergeThreads), 0, st, rows,
                     D, parts, po, plse, o, lse);
  return hipGetLastError();
}

}  // namespace xattn
