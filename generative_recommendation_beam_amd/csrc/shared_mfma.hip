// Shared stage on bf16 MFMA (xGR page, section 2.1 xAttention: the Shared
// cache holds the prompt once for all beams; the Shared stage computes local
// scores and max/sum statistics; matmul and softmax are fused). Because every
// beam of a request reads the same prompt KV, the B*G query rows of one
// (request, kv head) form a dense Q.K^T / P.V contraction: this kernel streams
// each prompt K/V tile from HBM into LDS once and lets all of the workgroup's
// query rows use it on the matrix cores.
//
// Work unit (one workgroup): (request r, kv head h, tile of 32*NW query rows,
// prompt split). Each wavefront owns 32 query rows and works in transposed
// form, S^T = K . Q^T and O^T += V^T . P^T, with v_mfma_f32_32x32x16_bf16:
//  - B operand of S^T: lane (hh = lane/32, c = lane%32) holds query row c,
//    head-dim elements [16*dc + 8*hh, +8) - loaded once, kept in registers;
//  - S^T accumulator: lane holds 16 keys of query column c, so the row max and
//    sum are lane-local except one exchange between the two lane halves;
//  - P^T (bf16) feeds the next MFMA straight from those registers; V^T is read
//    from an LDS copy whose key order is permuted to match.
// Online softmax with a lazy rescale: the running max used as the exponent
// offset only moves when a tile's max exceeds it by more than 8 (log2 units),
// which keeps every probability <= 256 and skips most output rescales; the
// result is exact either way because the final division uses the same offset.
// Optional epilogue (prompt split 0 only): fold in the beam's own generated
// tokens, gathered through its slot-table row (the Non-Shared stage), before
// normalizing, so the fused decode needs no separate merge when unsplit.
#include "device.h"
#include "kernels.h"

namespace xattn {

namespace {

constexpr int BN = 64;  // keys per tile

__device__ __forceinline__ int vt_pos(int key) {
  // Position of tile key `key` inside a V^T row: within each 16-key chunk the
  // keys held by lane half 0 of the P^T operand come first, then half 1.
  const int kk = key & 15;
  return (key & ~15) | (((kk >> 2) & 1) << 3) | ((kk >> 3) << 2) | (kk & 3);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void shared_mfma_kernel(SharedMfmaArgs a, int64_t n_logical) {
  constexpr int NT = NW * 64;
  constexpr int KSTR = D + 8;   // bf16 per K row in LDS (row = 16-byte multiple, padded)
  constexpr int VSTR = BN + 8;  // bf16 per V^T row in LDS
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int DCH = D / 8;    // 16-byte chunks per K/V row
  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VSTR];

  const int64_t lb = xcd_logical_block(blockIdx.x, gridDim.x, n_logical);
  if (lb < 0) return;  // uniform per workgroup
  const Shape& s = a.s;
  const int tile = (int)(lb % a.row_tiles);
  const int64_t t2 = lb / a.row_tiles;
  const int split = (int)(t2 % a.p_splits);
  const int pair = (int)(t2 / a.p_splits);
  const int h = pair % s.Hkv;
  const int r = pair / s.Hkv;
  const int G = s.Hq / s.Hkv;
  const int M = s.B * G;
  const float c = s.scale_log2;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;
  const int ql = lane & 31;

  const int row = tile * (NW * 32) + wave * 32 + ql;
  const bool row_ok = row < M;
  const int bq = row_ok ? row / G : 0;
  const int gq = row_ok ? row - bq * G : 0;
  const int64_t qrow = ((int64_t)r * s.B + bq) * s.Hq + h * G + gq;

  bf16x8_t qf[NDC];
  {
    const uint16_t* qp = a.q + qrow * D + 8 * hh;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (row_ok) u = *reinterpret_cast<const uint4*>(qp + 16 * dc);
      qf[dc] = __builtin_bit_cast(bf16x8_t, u);
    }
  }

  const int P = a.prefix_len[r];
  const int64_t kvbase = ((int64_t)h * s.n_ptok + a.prefix_off[r]) * D;
  const uint16_t* Kg = a.k_shared + kvbase;
  const uint16_t* Vg = a.v_shared + kvbase;
  const int kbeg = split * a.p_chunk;
  const int kend = min(P, kbeg + a.p_chunk);

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = neg_inf();
  float l_part = 0.f;

  for (int k0 = kbeg; k0 < kend; k0 += BN) {
    const int nvalid = min(BN, kend - k0);
    __syncthreads();  // every wavefront is done with the previous tile
    // K tile: row-major [key][d], coalesced 16-byte pieces.
    for (int i = tid; i < BN * DCH; i += NT) {
      const int key = i / DCH, ch = i - key * DCH;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (key < nvalid) v = *reinterpret_cast<const uint4*>(Kg + (int64_t)(k0 + key) * D + ch * 8);
      *reinterpret_cast<uint4*>(&sK[key * KSTR + ch * 8]) = v;
    }
    // V tile, transposed to [d][permuted key]: each thread packs a key pair
    // (2k, 2k+1) per head-dim element into one 32-bit LDS word.
    for (int i = tid; i < (BN / 2) * DCH; i += NT) {
      const int kp = i & (BN / 2 - 1), ch = i / (BN / 2);
      const int k_even = 2 * kp;
      uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
      if (k_even < nvalid) v0 = *reinterpret_cast<const uint4*>(Vg + (int64_t)(k0 + k_even) * D + ch * 8);
      if (k_even + 1 < nvalid) v1 = *reinterpret_cast<const uint4*>(Vg + (int64_t)(k0 + k_even + 1) * D + ch * 8);
      const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w};
      const uint32_t w1[4] = {v1.x, v1.y, v1.z, v1.w};
      const int pos = vt_pos(k_even);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (e & 1) ? (w0[e >> 1] >> 16) : (w0[e >> 1] & 0xffffu);
        const uint32_t hi = (e & 1) ? (w1[e >> 1] & 0xffff0000u) : (w1[e >> 1] << 16);
        *reinterpret_cast<uint32_t*>(&sV[(ch * 8 + e) * VSTR + pos]) = lo | hi;
      }
    }
    __syncthreads();

    // S^T = K . Q^T for two 32-key blocks.
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(&sK[(kb * 32 + ql) * KSTR + 16 * dc + 8 * hh]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[dc], sacc[kb], 0, 0, 0);
      }
    }
    // scale into log2 units, mask keys past the end, tile max per query
    float mx = neg_inf();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
        const float v = key < nvalid ? sacc[kb][i] * c : neg_inf();
        sacc[kb][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__any(mx > m_run + 8.0f)) {
      const float mn = fmaxf(m_run, mx);
      const float alpha = exp2_approx(m_run - mn);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      l_part *= alpha;
      m_run = mn;
    }
    bf16x8_t pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2_approx(sacc[kb][i] - m_run);
        l_part += p;
        pf[2 * kb + (i >> 3)][i & 7] = (__bf16)p;
      }
    // O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(&sV[(32 * db + ql) * VSTR + 16 * cc + 8 * hh]);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[cc], oacc[db], 0, 0, 0);
      }
  }

  // Non-Shared epilogue: the beam's own generated tokens (split 0 only).
  if (a.k_pool != nullptr && split == 0) {
    const int L = a.unshared_len[r];
    const int64_t n = (int64_t)r * s.B + bq;
    const int32_t* trow = a.slot_table + n * s.T_max;
    for (int t = 0; t < L; ++t) {
      const int64_t slot = trow[t];
      const uint16_t* kp = a.k_pool + (slot * s.Hkv + h) * D;
      float dot = 0.f;
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        const uint4 u = *reinterpret_cast<const uint4*>(kp + 16 * dc + 8 * hh);
        const bf16x8_t kk = __builtin_bit_cast(bf16x8_t, u);
#pragma unroll
        for (int j = 0; j < 8; ++j) dot += (float)qf[dc][j] * (float)kk[j];
      }
      dot += __shfl_xor(dot, 32);
      const float st = dot * c;
      if (st > m_run) {
        const float alpha = exp2_approx(m_run - st);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        l_part *= alpha;
        m_run = st;
      }
      const float p = exp2_approx(st - m_run);
      if (hh == 0) l_part += p;
      const uint16_t* vp = a.v_pool + (slot * s.Hkv + h) * D + 4 * hh;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const uint2 u = *reinterpret_cast<const uint2*>(vp + 32 * db + 8 * ig);
          oacc[db][4 * ig + 0] += p * bf16_bits_to_f32(u.x & 0xffffu);
          oacc[db][4 * ig + 1] += p * __uint_as_float(u.x & 0xffff0000u);
          oacc[db][4 * ig + 2] += p * bf16_bits_to_f32(u.y & 0xffffu);
          oacc[db][4 * ig + 3] += p * __uint_as_float(u.y & 0xffff0000u);
        }
    }
  }

  const float l_tot = l_part + __shfl_xor(l_part, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  float* ob = a.out.o;
  float* lbp = a.out.lse;
  if (a.out.part_stride) {
    const int64_t part = a.out.part_base + split;
    ob += part * a.out.part_stride * D;
    lbp += part * a.out.part_stride;
  }
  float* dst = ob + qrow * D + 4 * hh;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig)
      *reinterpret_cast<float4*>(dst + 32 * db + 8 * ig) =
          make_float4(oacc[db][4 * ig] * inv, oacc[db][4 * ig + 1] * inv,
                      oacc[db][4 * ig + 2] * inv, oacc[db][4 * ig + 3] * inv);
  if (lbp && hh == 0) lbp[qrow] = l_tot > 0.f ? (m_run + log2_approx(l_tot)) * kLn2 : neg_inf();
}

template <int D>
hipError_t launch_d(const SharedMfmaArgs& a, hipStream_t st) {
  const int64_t n_logical = (int64_t)a.s.R * a.s.Hkv * a.p_splits * a.row_tiles;
  if (n_logical == 0) return hipSuccess;
  const int64_t grid = (n_logical + 7) / 8 * 8;
  switch (a.waves) {
    case 1: hipLaunchKernelGGL((shared_mfma_kernel<D, 1>), dim3((unsigned)grid), dim3(64), 0, st, a, n_logical); break;
    case 2: hipLaunchKernelGGL((shared_mfma_kernel<D, 2>), dim3((unsigned)grid), dim3(128), 0, st, a, n_logical); break;
    default: hipLaunchKernelGGL((shared_mfma_kernel<D, 4>), dim3((unsigned)grid), dim3(256), 0, st, a, n_logical); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_shared_mfma(const SharedMfmaArgs& a, hipStream_t st) {
  return a.s.D == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace xattn
