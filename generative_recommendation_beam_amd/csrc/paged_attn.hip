// PagedAttention-style per-beam decode attention: the comparison baseline.
//
// The xGR page (section 1) names what its split cache avoids: serving systems
// in the PagedAttention mould treat every beam as its own sequence, so each
// beam reads the shared prompt again through its block table, and a beam that
// branches needs its partially filled blocks copied. This kernel computes the
// same attention that way, on a block-paged cache: K/V in blocks of
// kPagedBlock tokens, [num_blocks][H_kv][kPagedBlock][D] bf16, and per beam a
// block table [N_b][max_blocks] and a length seq_len[N_b] (prompt + its own
// generated tokens). It is a fair baseline, not a strawman: wide loads, every
// kv head's query group served by one pass over the blocks, and the sequence
// split into partitions merged with the log-sum-exp rule.
//
// One workgroup (4 waves) per (beam, kv head, group of up to 4 query heads,
// partition of kPagedPart tokens). Wave w takes blocks w, w+4, ... of the
// partition. A wave's 64 lanes are 8 token slots of 8 lanes; the 8 lanes of a
// slot hold D/8 elements of one key, so a score needs a 3-step shuffle sum.
// Each slot keeps its own online-softmax state; slots, then waves (through
// LDS), are combined at the end.
#include "device.h"
#include "kernels.h"

namespace xattn {

namespace {

constexpr int kWaves = 4;
constexpr int kNG = 4;  // query heads per unit

template <int D>
__global__ __launch_bounds__(kWaves * 64) void paged_attn_kernel(PagedArgs a, int64_t n_units) {
  constexpr int EPL = D / 8;
  __shared__ float xm[kWaves][kNG], xl[kWaves][kNG];
  __shared__ float xo[kWaves][kNG][D];
  const int64_t unit = blockIdx.x;
  if (unit >= n_units) return;  // uniform
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane >> 3, dl = lane & 7;
  const int G = a.Hq / a.Hkv;
  const int ngroups = (G + kNG - 1) / kNG;
  int64_t u = unit;
  const int part = (int)(u % a.nparts);
  u /= a.nparts;
  const int grp = (int)(u % ngroups);
  u /= ngroups;
  const int h = (int)(u % a.Hkv);
  const int64_t n = u / a.Hkv;
  const int g0 = grp * kNG;
  const int ng = min(kNG, G - g0);

  float q[kNG][EPL], acc[kNG][EPL], m[kNG], l[kNG];
  {
    const uint16_t* qb = a.q + ((n * a.Hq) + h * G + g0) * (int64_t)D + dl * EPL;
#pragma unroll
    for (int g = 0; g < kNG; ++g) {
      float t[EPL];
      if (g < ng) {
#pragma unroll
        for (int e = 0; e < EPL; e += 8) Load<uint16_t, 8>::run(qb + (int64_t)g * D + e, t + e);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) t[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        q[g][e] = t[e] * a.scale_log2;
        acc[g][e] = 0.f;
      }
      m[g] = neg_inf();
      l[g] = 0.f;
    }
  }

  const int len = a.seq_len[n];
  const int t_begin = part * kPagedPart;
  const int t_end = min(len, t_begin + kPagedPart);
  const int32_t* btab = a.block_table + n * (int64_t)a.max_blocks;
  for (int blk = t_begin / kPagedBlock + wave; blk * kPagedBlock < t_end; blk += kWaves) {
    const int64_t pb = btab[blk];
    const uint16_t* kb = a.k_cache + ((pb * a.Hkv + h) * kPagedBlock) * (int64_t)D + dl * EPL;
    const uint16_t* vb = a.v_cache + ((pb * a.Hkv + h) * kPagedBlock) * (int64_t)D + dl * EPL;
    float kv[2][EPL], vv[2][EPL];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int tk = half * 8 + slot;  // token within the block
#pragma unroll
      for (int e = 0; e < EPL; e += 8) {
        Load<uint16_t, 8>::run(kb + (int64_t)tk * D + e, kv[half] + e);
        Load<uint16_t, 8>::run(vb + (int64_t)tk * D + e, vv[half] + e);
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int tok = blk * kPagedBlock + half * 8 + slot;
      const bool valid = tok >= t_begin && tok < t_end;
      float sc[kNG];
#pragma unroll
      for (int g = 0; g < kNG; ++g) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s += q[g][e] * kv[half][e];
        sc[g] = s;
      }
#pragma unroll
      for (int off = 1; off <= 4; off <<= 1)
#pragma unroll
        for (int g = 0; g < kNG; ++g) sc[g] += __shfl_xor(sc[g], off);
      if (valid) {
#pragma unroll
        for (int g = 0; g < kNG; ++g) {
          const float mn = fmaxf(m[g], sc[g]);
          const float alpha = exp2_approx(m[g] - mn);  // m = -inf -> 0
          const float p = exp2_approx(sc[g] - mn);
          l[g] = l[g] * alpha + p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] = acc[g][e] * alpha + p * vv[half][e];
          m[g] = mn;
        }
      }
    }
  }

  // Combine the 8 token slots (lanes 8, 16, 32 apart).
#pragma unroll
  for (int off = 8; off <= 32; off <<= 1) {
#pragma unroll
    for (int g = 0; g < kNG; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float a1 = m[g] == neg_inf() ? 0.f : exp2_approx(m[g] - mn);
      const float a2 = mo == neg_inf() ? 0.f : exp2_approx(mo - mn);
      l[g] = l[g] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = acc[g][e] * a1 + __shfl_xor(acc[g][e], off) * a2;
      m[g] = mn;
    }
  }
  // Then the 4 waves, through LDS.
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < kNG; ++g) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) xo[wave][g][dl * EPL + e] = acc[g][e];
      if (dl == 0) {
        xm[wave][g] = m[g];
        xl[wave][g] = l[g];
      }
    }
  }
  __syncthreads();
  if (wave != 0 || slot != 0) return;
  const int64_t row0 = n * a.Hq + h * G + g0;
  float* ob = a.o;
  float* lb = a.lse;
  if (a.nparts > 1) {
    ob = a.part_o + (int64_t)part * a.rows * D;
    lb = a.part_lse + (int64_t)part * a.rows;
  }
#pragma unroll
  for (int g = 0; g < kNG; ++g) {
    if (g >= ng) break;
    float mx = neg_inf();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, xm[w][g]);
    float lt = 0.f, o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = xm[w][g] == neg_inf() ? 0.f : exp2_approx(xm[w][g] - mx);
      lt += xl[w][g] * wt;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] += xo[w][g][dl * EPL + e] * wt;
    }
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    float* dst = ob + (row0 + g) * D + dl * EPL;
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      *reinterpret_cast<float4*>(dst + e) = make_float4(o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv);
    if (lb && dl == 0) lb[row0 + g] = lt > 0.f ? (mx + log2_approx(lt)) * kLn2 : neg_inf();
  }
}

// Copy whole blocks (all kv heads) src[i] -> dst[i]: the copies a branching
// beam needs in a block-paged cache. 16-byte pieces, grid-strided.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint16_t* kc, uint16_t* vc, const int32_t* src,
                                                          const int32_t* dst, int n, int64_t block_elems) {
  const int64_t pieces = block_elems / 8;  // 8 bf16 per 16 bytes
  const int64_t total = pieces * n;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i / pieces, k = i - b * pieces;
    const int64_t so = (int64_t)src[b] * block_elems + k * 8, d = (int64_t)dst[b] * block_elems + k * 8;
    *reinterpret_cast<uint4*>(kc + d) = *reinterpret_cast<const uint4*>(kc + so);
    *reinterpret_cast<uint4*>(vc + d) = *reinterpret_cast<const uint4*>(vc + so);
  }
}

}  // namespace

hipError_t launch_paged_attn(const PagedArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int64_t n_units = a.rows / a.Hq * a.Hkv * ((G + kNG - 1) / kNG) * a.nparts;
  if (n_units == 0) return hipSuccess;
  if (a.D == 64)
    hipLaunchKernelGGL(paged_attn_kernel<64>, dim3((unsigned)n_units), dim3(kWaves * 64), 0, st, a, n_units);
  else
    hipLaunchKernelGGL(paged_attn_kernel<128>, dim3((unsigned)n_units), dim3(kWaves * 64), 0, st, a, n_units);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nparts == 1) return e;
  return launch_merge_parts(a.rows, a.D, a.nparts, a.part_o, a.part_lse, a.o, a.lse, st);
}

hipError_t launch_copy_blocks(uint16_t* kc, uint16_t* vc, const int32_t* src, const int32_t* dst, int n,
                              int64_t block_elems, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t total = block_elems / 8 * n;
  int64_t grid = (total + 255) / 256;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(256), 0, st, kc, vc, src, dst, n, block_elems);
  return hipGetLastError();
}

}  // namespace xattn
