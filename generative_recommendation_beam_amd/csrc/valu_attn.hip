// Vector-ALU attention of a few query rows over a key range (no MFMA).
//
// Used for the Non-Shared stage (xGR page, section 2.1 xAttention: each beam
// attends to its own generated tokens, gathered through its slot-table row
// from the token-granular pool) and for the fp32 path.
// The Non-Shared work is bandwidth-bound and tiny per beam: a GEMV, not a
// contraction worth the matrix cores.
//
// One wavefront owns one unit = (beam n, kv head h, group of up to NG query
// heads of that kv head, key split). Its 64 lanes form 4 key slots of 16
// lanes; a slot's 16 lanes hold one key row (D/16 elements each), so a key
// costs one 16-lane shuffle reduction per query row. Each slot keeps its own
// online-softmax state (max, sum, output) over the keys it saw; the 4 slots
// are combined at the end with the same log-sum-exp rule as the Merge stage.
//
// Keys go in batches of U steps (4U keys): the K/V rows of a whole batch are
// requested before any of them is used, and the slot indices of the next
// batch of generated tokens are requested beside the current batch's rows,
// so a wave waits one memory round trip per batch rather than per step.
#include "device.h"
#include "kernels.h"

namespace xattn {

namespace {

constexpr int kValuWaves = 4;
constexpr int kValuWgMax = kValuWgMaxSplits;
constexpr int kValuFoldChunk = 4;  // folded partials whose loads are in flight together

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over a key slot's 16 lanes (one DPP row), every lane getting the same
// bits: the butterfly over lane distances 8, 4, 2, 1, with the first two as
// row rotations (equal to the exchanges once the partial sums are symmetric)
// and the last two as quad permutations. Register-to-register, no LDS.
__device__ __forceinline__ float slot_sum(float x) {
  x += dpp_f32<0x128>(x);  // row_ror:8 (lane i ^ 8)
  x += dpp_f32<0x124>(x);  // row_ror:4 (x now symmetric under i ^ 8)
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1] (lane i ^ 2)
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2] (lane i ^ 1)
  return x;
}

// The value of lane i ^ LM (LM = 16 or 32) through the gfx950 lane swaps,
// register to register. The whole wavefront must be active.
template <int LM>
__device__ __forceinline__ float xor_far(float x, int lane) {
  const uint32_t v = __builtin_bit_cast(uint32_t, x);
  if constexpr (LM == 16) {  // odd 16-lane rows of one copy swapped with even rows of the other
    const auto w = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return __builtin_bit_cast(float, (lane & 16) ? w[0] : w[1]);
  } else {  // upper 32 lanes of one copy swapped with the lower 32 of the other
    const auto w = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __builtin_bit_cast(float, (lane & 32) ? w[0] : w[1]);
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// One lane's share (EPL elements) of a key or query row as the score needs
// it: bf16 rows stay as loaded, two elements per dword, for the packed bf16
// dot product (products exact, sums in fp32); fp32 rows as floats.
template <typename T, int EPL>
struct KRow;
template <int EPL>
struct KRow<uint16_t, EPL> {
  uint32_t w[EPL / 2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    if constexpr (EPL == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      w[0] = v.x;
      w[1] = v.y;
      w[2] = v.z;
      w[3] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      w[0] = v.x;
      w[1] = v.y;
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i) w[i] = 0u;
  }
  __device__ __forceinline__ float dot(const KRow& k) const {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i)
      a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[i]), __builtin_bit_cast(bf16x2_t, k.w[i]), a,
                                          false);
    return a;
  }
};
template <int EPL>
struct KRow<float, EPL> {
  float f[EPL];
  __device__ __forceinline__ void load(const float* p) { Load<float, EPL>::run(p, f); }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int e = 0; e < EPL; ++e) f[e] = 0.f;
  }
  __device__ __forceinline__ float dot(const KRow& k) const {
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a += f[e] * k.f[e];
    return a;
  }
};

template <typename T, int D, int NG, bool BATCH>
struct ValuState {
  static constexpr int EPL = D / 16;
  // Four bf16 query heads: during the walk the heads are spread over a key
  // slot's 16 lanes. Lane i of a slot belongs to head group c = (i / 4) % 4
  // and holds its heads in the order c, c+1, c+2, c+3 (mod 4): q[j] and
  // acc[j] are head (c + j) & 3. A score's 16-lane sum then reduces all four
  // heads at once (each level adds the partner's copy of the heads this lane
  // keeps: 2 + 1 + 2 row operations instead of 4 per head), every lane ends
  // with the full score of head c, which only it (and its group) turns into
  // a weight, and the four weights reach every lane by three row rotations.
  // m[0] / l[0] are head c's; to_absolute() restores the plain layout.
  static constexpr bool REL = BATCH && NG == 4 && sizeof(T) == 2;
  KRow<T, EPL> q[NG];  // bf16: as loaded; fp32: pre-scaled by scale_log2
  float qscale;        // applied to each bf16 score (the fp32 q carries it)
  float m[NG], l[NG];
  float acc[NG][EPL];

  // head group of this lane within its key slot
  __device__ __forceinline__ static int head_group(int lane) { return (lane >> 2) & 3; }
  // the values of heads c+1, c+2, c+3 from the lanes of those head groups
  // (lane i reads lane i+4, i+8, i+12 of its 16-lane row)
  __device__ __forceinline__ static void spread(float x, float* out) {
    out[0] = x;
    out[1] = dpp_f32<0x12C>(x);  // row_ror:12 (lane i + 4)
    out[2] = dpp_f32<0x128>(x);  // row_ror:8  (lane i + 8)
    out[3] = dpp_f32<0x124>(x);  // row_ror:4  (lane i - 4)
  }

  // The plain layout after a walk in the head-group layout: m, l and acc per
  // absolute head in every lane.
  __device__ __forceinline__ void to_absolute(int lane) {
    if constexpr (REL) {
      const int c = head_group(lane);
      float mr[4], lr[4];
      spread(m[0], mr);
      spread(l[0], lr);
      float ar[4][EPL];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e) ar[j][e] = acc[j][e];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j = (g - c) & 3;  // head g sits at relative index j
        m[g] = j == 0 ? mr[0] : j == 1 ? mr[1] : j == 2 ? mr[2] : mr[3];
        l[g] = j == 0 ? lr[0] : j == 1 ? lr[1] : j == 2 ? lr[2] : lr[3];
#pragma unroll
        for (int e = 0; e < EPL; ++e)
          acc[g][e] = j == 0 ? ar[0][e] : j == 1 ? ar[1][e] : j == 2 ? ar[2][e] : ar[3][e];
      }
    }
  }

  // Batch update in the head-group layout (see update_batch). The value
  // rows stay as loaded (two bf16 elements per dword), and the weights go
  // in pairs of steps: the two steps' weights of a head are rounded to bf16
  // and packed, and one bf16 dot product per output element adds both
  // steps' weighted values (products exact, sums in fp32), after the two
  // steps' elements are paired up by byte permutes. The running sum adds
  // the rounded weights, the ones the values are weighted with.
  template <int U>
  __device__ __forceinline__ void update_batch_rel(const KRow<T, EPL>* kv, const KRow<T, EPL>* vr, int nvalid) {
    static_assert(U % 2 == 0, "steps go in pairs");
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) s4[j] = q[j].dot(kv[u]);
      // lanes i and i-8 (head groups c and c+2): keep heads c, c+1
      const float t0 = s4[0] + dpp_f32<0x128>(s4[2]);
      const float t1 = s4[1] + dpp_f32<0x128>(s4[3]);
      // lane i-4 (group c-1) holds head c as its second: all four groups
      float x = t0 + dpp_f32<0x124>(t1);
      x += dpp_f32<0xB1>(x);  // quad_perm [1,0,3,2]
      x += dpp_f32<0x4E>(x);  // quad_perm [2,3,0,1]
      sc[u] = fminf(x * qscale, u < nvalid ? __builtin_inff() : neg_inf());
    }
    float mx = sc[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u]);
    const bool mv = mx > m[0] + 8.0f;
    if (__any(mv)) {  // rare after the first batch
      const float mn = mv ? mx : m[0];
      const float alpha = mv ? exp2_approx(m[0] - mn) : 1.0f;  // m = -inf -> 0
      l[0] *= alpha;
      m[0] = mn;
      float ar[4];
      spread(alpha, ar);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] *= ar[j];
    }
    const float mref = m[0] == neg_inf() ? 0.f : m[0];
#pragma unroll
    for (int u = 0; u < U; u += 2) {
      const bf16x2_t pk{(__bf16)exp2_approx(sc[u] - mref), (__bf16)exp2_approx(sc[u + 1] - mref)};
      const uint32_t pb = __builtin_bit_cast(uint32_t, pk);
      l[0] += __uint_as_float(pb << 16) + __uint_as_float(pb & 0xffff0000u);
      float pr[4];
      spread(__uint_as_float(pb), pr);
#pragma unroll
      for (int i = 0; i < EPL / 2; ++i) {
        // element 2i of steps u and u+1, then element 2i+1 of both
        const uint32_t ev = __builtin_amdgcn_perm(vr[u + 1].w[i], vr[u].w[i], 0x05040100u);
        const uint32_t od = __builtin_amdgcn_perm(vr[u + 1].w[i], vr[u].w[i], 0x07060302u);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x2_t pj = __builtin_bit_cast(bf16x2_t, pr[j]);
          acc[j][2 * i] = __builtin_amdgcn_fdot2_f32_bf16(pj, __builtin_bit_cast(bf16x2_t, ev), acc[j][2 * i], false);
          acc[j][2 * i + 1] =
              __builtin_amdgcn_fdot2_f32_bf16(pj, __builtin_bit_cast(bf16x2_t, od), acc[j][2 * i + 1], false);
        }
      }
    }
  }

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      m[g] = neg_inf();
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }
  }

  // A batch of U steps, each over the 4 keys held by the 4 slots: kv[u] /
  // vv[u] are this lane's D/16 elements of its slot's key and value rows in
  // step u; step u holds a key for this slot iff u < nvalid. The scores of
  // the whole batch come first; the reference maximum then moves at most
  // once per batch (lazily: only when a score passes it by more than 8, in
  // log2 units, so every weight stays below 2^8), and the weights and value
  // updates follow as straight-line code.
  template <int U>
  __device__ __forceinline__ void update_batch(const KRow<T, EPL>* kv, const float (*vv)[EPL], int nvalid) {
    float s[U][NG];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < NG; ++g) s[u][g] = sizeof(T) == 2 ? q[g].dot(kv[u]) * qscale : q[g].dot(kv[u]);
    // Steps past nvalid get -inf through a min with a bound chosen apart from
    // the sums (a select would let the compiler branch around them).
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float bound = u < nvalid ? __builtin_inff() : neg_inf();
#pragma unroll
      for (int g = 0; g < NG; ++g) s[u][g] = fminf(slot_sum(s[u][g]), bound);
    }
    bool move = false;
    float mx[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      mx[g] = s[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) mx[g] = fmaxf(mx[g], s[u][g]);
      move |= mx[g] > m[g] + 8.0f;
    }
    if (__any(move)) {  // rare after the first batch
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const bool mv = mx[g] > m[g] + 8.0f;
        const float mn = mv ? mx[g] : m[g];
        const float alpha = mv ? exp2_approx(m[g] - mn) : 1.0f;  // m = -inf -> 0
        l[g] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
        m[g] = mn;
      }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      // a slot with no key yet keeps m = -inf and only -inf scores: weight 0
      const float mref = m[g] == neg_inf() ? 0.f : m[g];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = exp2_approx(s[u][g] - mref);
        l[g] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] += p * vv[u][e];
      }
    }
  }

  // One step over the 4 keys held by the 4 slots: kv / vv are this lane's
  // D/16 elements of its slot's key and value rows; `valid` is uniform per
  // slot.
  __device__ __forceinline__ void update(const KRow<T, EPL>& kv, const float* vv, bool valid) {
    float s[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) s[g] = sizeof(T) == 2 ? q[g].dot(kv) * qscale : q[g].dot(kv);
#pragma unroll
    for (int g = 0; g < NG; ++g) s[g] = slot_sum(s[g]);
    if (valid) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        // Lazy rescale: the reference maximum moves only when a score passes
        // it by more than 8 (log2 units), so every weight stays below 2^8 and
        // most steps skip the accumulator rescale. The 16 lanes of a key slot
        // hold the same bits, so the choice is the same across them.
        if (__any(s[g] > m[g] + 8.0f)) {
          const float mn = fmaxf(m[g], s[g]);
          const float alpha = exp2_approx(m[g] - mn);  // m = -inf -> 0
          l[g] *= alpha;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
          m[g] = mn;
        }
        const float p = exp2_approx(s[g] - m[g]);
        l[g] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] += p * vv[e];
      }
    }
  }

  // Combine the 4 key slots (lanes 16 and 32 apart).
  __device__ __forceinline__ void combine_slots(int lane) {
    combine_with<16>(lane);
    combine_with<32>(lane);
  }
  template <int off>
  __device__ __forceinline__ void combine_with(int lane) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const float mo = xor_far<off>(m[g], lane);
      const float lo = xor_far<off>(l[g], lane);
      const float mn = fmaxf(m[g], mo);
      const float a1 = (m[g] == neg_inf()) ? 0.f : exp2_approx(m[g] - mn);
      const float a2 = (mo == neg_inf()) ? 0.f : exp2_approx(mo - mn);
      l[g] = l[g] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = xor_far<off>(acc[g][e], lane);
        acc[g][e] = acc[g][e] * a1 + ao * a2;
      }
      m[g] = mn;
    }
  }
};

// WGM: the splits of one (beam, kv head, head group) are the waves of one
// workgroup (wave w = split w) and are merged there, in split order, into the
// final output; otherwise kValuWaves consecutive units per workgroup.
template <typename T, int D, int NG, bool WGM, bool BATCH>
__global__ __launch_bounds__(WGM ? kValuWgMax * 64 : kValuWaves * 64) void valu_attn_kernel(
    ValuArgs a, int64_t n_units, int ngroups) {
  constexpr int EPL = D / 16;
  // Steps per batch: 64 dwords of K/V rows in flight per lane at most (32
  // with 8 query heads, whose state takes twice the registers), 8 steps at
  // most.
  constexpr int STEP_DW = 2 * EPL * (int)sizeof(T) / 4;
  constexpr int BUF_DW = NG >= 8 ? 32 : 64;
  constexpr int U = BUF_DW / STEP_DW < 8 ? BUF_DW / STEP_DW : 8;
  const int lane = threadIdx.x & 63;
  const int64_t unit = (int64_t)blockIdx.x * (WGM ? a.splits : kValuWaves) + (threadIdx.x >> 6);
  if (unit >= n_units) return;  // uniform per wavefront
  const Shape& s = a.s;
  int64_t u = unit;
  const int split = (int)(u % a.splits);
  u /= a.splits;
  const int grp = (int)(u % ngroups);
  u /= ngroups;
  const int h = (int)(u % s.Hkv);
  const int64_t n = u / s.Hkv;
  const int r = (int)(n / s.B);
  const int G = s.Hq / s.Hkv;
  const int g0 = grp * NG;
  const int ng = min(NG, G - g0);
  const int slot_id = lane >> 4;
  const int dl = lane & 15;

  ValuState<T, D, NG, BATCH> st;
  st.init();
  {
    const T* qb = static_cast<const T*>(a.q) + ((n * s.Hq) + h * G + g0) * (int64_t)D + dl * EPL;
    st.qscale = s.scale_log2;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int g = decltype(st)::REL ? (st.head_group(lane) + j) & 3 : j;  // head of q[j]
      if (g < ng)
        st.q[j].load(qb + (int64_t)g * D);
      else
        st.q[j].zero();
      if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.q[j].f[e] *= s.scale_log2;
      }
    }
  }

  if (a.use_prefix) {
    const int P = a.prefix_len[r];
    int k0 = 0, k1 = P;
    if (!a.use_gen || a.splits > 1) {
      k0 = split * a.chunk;
      k1 = min(P, k0 + a.chunk);
    }
    const T* kb = static_cast<const T*>(a.k_shared) + ((int64_t)h * s.n_ptok + a.prefix_off[r]) * D + dl * EPL;
    const T* vb = static_cast<const T*>(a.v_shared) + ((int64_t)h * s.n_ptok + a.prefix_off[r]) * D + dl * EPL;
    for (int j0 = k0; j0 < k1; j0 += 4 * U) {
      KRow<T, EPL> kv[U];
      if constexpr (decltype(st)::REL) {  // value rows as loaded
        KRow<T, EPL> vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {  // keys past k1 read row k1-1 and are skipped
          const int64_t jj = min(j0 + 4 * u + slot_id, k1 - 1);
          kv[u].load(kb + jj * D);
          vr[u].load(vb + jj * D);
        }
        st.template update_batch_rel<U>(kv, vr, (k1 - j0 - slot_id + 3) / 4);
        continue;
      }
      float vv[U][EPL];
#pragma unroll
      for (int u = 0; u < U; ++u) {  // keys past k1 read row k1-1 and are skipped
        const int64_t jj = min(j0 + 4 * u + slot_id, k1 - 1);
        kv[u].load(kb + jj * D);
        Load<T, EPL>::run(vb + jj * D, vv[u]);
      }
      if constexpr (BATCH) {
        st.template update_batch<U>(kv, vv, (k1 - j0 - slot_id + 3) / 4);
      } else {  // short runs and fp32: per-step updates, invalid steps skipped
#pragma unroll
        for (int u = 0; u < U; ++u) st.update(kv[u], vv[u], j0 + 4 * u + slot_id < k1);
      }
    }
  }
  if (a.use_gen && (!a.use_prefix || split == 0)) {  // beside a split prompt: in split 0
    const int L = a.unshared_len[r];
    int t0 = 0, t1 = L;
    if (!a.use_prefix) {
      t0 = split * a.chunk;
      t1 = min(L, t0 + a.chunk);
    }
    if (t1 > t0) {
      const int32_t* trow = a.slot_table + n * s.T_max;
      const T* kp = static_cast<const T*>(a.k_pool) + h * D + dl * EPL;
      const T* vp = static_cast<const T*>(a.v_pool) + h * D + dl * EPL;
      const int64_t tok_stride = (int64_t)s.Hkv * D;
      // Tokens past t1 read the slot of token t1-1 and are skipped.
      int slot[U];
#pragma unroll
      for (int u = 0; u < U; ++u) slot[u] = trow[min(t0 + 4 * u + slot_id, t1 - 1)];
      for (int j0 = t0; j0 < t1; j0 += 4 * U) {
        KRow<T, EPL> kv[U];
        if constexpr (decltype(st)::REL) {  // value rows as loaded
          {
            // Issue priority falls as the walk advances (3, then 2, 1 and 0
            // past a half, three quarters and seven eighths of the tokens):
            // the workgroups sharing a SIMD finish closer together. Measured
            // on MI355X (4 requests x 16 beams, 512-token tails): 47.2 ->
            // 46.2 us per append + decode call.
            const int rem = t1 - j0, tot = t1 - t0;  // uniform
            if (rem * 2 > tot) __builtin_amdgcn_s_setprio(3);
            else if (rem * 4 > tot) __builtin_amdgcn_s_setprio(2);
            else if (rem * 8 > tot) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
          }
          KRow<T, EPL> vr[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            kv[u].load(kp + slot[u] * tok_stride);
            vr[u].load(vp + slot[u] * tok_stride);
          }
#pragma unroll
          for (int u = 0; u < U; ++u) slot[u] = trow[min(j0 + 4 * U + 4 * u + slot_id, t1 - 1)];
          st.template update_batch_rel<U>(kv, vr, (t1 - j0 - slot_id + 3) / 4);
          continue;
        }
        float vv[U][EPL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          kv[u].load(kp + slot[u] * tok_stride);
          Load<T, EPL>::run(vp + slot[u] * tok_stride, vv[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) slot[u] = trow[min(j0 + 4 * U + 4 * u + slot_id, t1 - 1)];
        if constexpr (BATCH) {
          st.template update_batch<U>(kv, vv, (t1 - j0 - slot_id + 3) / 4);
        } else {
#pragma unroll
          for (int u = 0; u < U; ++u) st.update(kv[u], vv[u], j0 + 4 * u + slot_id < t1);
        }
      }
    }
  }
  if constexpr (decltype(st)::REL) __builtin_amdgcn_s_setprio(0);
  st.to_absolute(lane);
  st.combine_slots(lane);
  // The wave (split) that finalizes query head g of the group.
  auto owner = [&](int g) { return (WGM && a.fold_parts > 0) ? g % a.splits : 0; };

  if constexpr (WGM) {  // the grid holds exactly n_units waves: all reach the barrier
    __shared__ float s_ml[kValuWgMax][NG][2];
    __shared__ float s_acc[kValuWgMax][NG][D];
    if (slot_id == 0) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_acc[split][g][dl * EPL + e] = st.acc[g][e];
        if (dl == 0) {
          s_ml[split][g][0] = st.m[g];
          s_ml[split][g][1] = st.l[g];
        }
      }
    }
    __syncthreads();
    // Wave w finalizes the query heads g with g % splits == w (without a
    // fold, wave 0 takes them all: the order of the writes does not matter).
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (owner(g) != split) continue;  // uniform per wavefront
      float mt = neg_inf();
      for (int w = 0; w < a.splits; ++w) mt = fmaxf(mt, s_ml[w][g][0]);
      float lt = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) st.acc[g][e] = 0.f;
      for (int w = 0; w < a.splits; ++w) {
        const float mw = s_ml[w][g][0];
        const float sc = mw == neg_inf() ? 0.f : exp2_approx(mw - mt);
        lt += s_ml[w][g][1] * sc;
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.acc[g][e] += s_acc[w][g][dl * EPL + e] * sc;
      }
      st.m[g] = mt;
      st.l[g] = lt;
    }
  }
  if (slot_id != 0) return;
  const int64_t row0 = n * s.Hq + h * G + g0;
  if (a.fold_parts > 0) {
    // Fold the earlier launch's partials (normalized O, natural-log lse) into
    // this state: a partial weighs 2^(lse*log2(e) - m) against the new offset
    // m. kValuFoldChunk partials' loads are in flight together.
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g >= ng) break;
      if (owner(g) != split) continue;  // uniform per wavefront
      const int64_t row = row0 + g;
      for (int p0 = 0; p0 < a.fold_parts; p0 += kValuFoldChunk) {
        float lp[kValuFoldChunk];
        float4 ov[kValuFoldChunk][EPL / 4];
#pragma unroll
        for (int q = 0; q < kValuFoldChunk; ++q) {
          const int p = min(p0 + q, a.fold_parts - 1);  // past the last: a repeat, weight 0 below
          lp[q] = a.fold_lse[p * a.fold_stride + row] * kLog2e;
          const float* po = a.fold_o + (p * a.fold_stride + row) * D + dl * EPL;
#pragma unroll
          for (int e = 0; e < EPL / 4; ++e) ov[q][e] = *reinterpret_cast<const float4*>(po + 4 * e);
        }
        float mt = st.m[g];
#pragma unroll
        for (int q = 0; q < kValuFoldChunk; ++q)
          if (p0 + q < a.fold_parts) mt = fmaxf(mt, lp[q]);
        const float sc = (mt == neg_inf() || st.m[g] == neg_inf()) ? 0.f : exp2_approx(st.m[g] - mt);
        float lt = st.l[g] * sc;
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.acc[g][e] *= sc;
#pragma unroll
        for (int q = 0; q < kValuFoldChunk; ++q) {
          const float wgt =
              (p0 + q >= a.fold_parts || mt == neg_inf() || lp[q] == neg_inf()) ? 0.f : exp2_approx(lp[q] - mt);
          lt += wgt;
#pragma unroll
          for (int e = 0; e < EPL / 4; ++e) {
            st.acc[g][4 * e] += ov[q][e].x * wgt;
            st.acc[g][4 * e + 1] += ov[q][e].y * wgt;
            st.acc[g][4 * e + 2] += ov[q][e].z * wgt;
            st.acc[g][4 * e + 3] += ov[q][e].w * wgt;
          }
        }
        st.m[g] = mt;
        st.l[g] = lt;
      }
    }
  }
  float* ob = a.out.o;
  float* lb = a.out.lse;
  if (a.out.part_stride) {
    const int64_t part = a.out.part_base + split;
    ob += part * a.out.part_stride * D;
    lb += part * a.out.part_stride;
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (g >= ng) break;
    if (owner(g) != (WGM ? split : 0)) continue;  // uniform per wavefront
    const float l = st.l[g];
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    float* dst = ob + (row0 + g) * D + dl * EPL;
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      *reinterpret_cast<float4*>(dst + e) =
          make_float4(st.acc[g][e] * inv, st.acc[g][e + 1] * inv, st.acc[g][e + 2] * inv,
                      st.acc[g][e + 3] * inv);
    if (lb && dl == 0) lb[row0 + g] = l > 0.f ? (st.m[g] + log2_approx(l)) * kLn2 : neg_inf();
  }
}

template <typename T, int D, int NG, bool BATCH>
hipError_t launch_one(const ValuArgs& a, dim3 grid, dim3 block, bool wgm, int64_t units, int ngroups,
                      hipStream_t st) {
  if (wgm)
    hipLaunchKernelGGL((valu_attn_kernel<T, D, NG, true, BATCH>), grid, block, 0, st, a, units, ngroups);
  else
    hipLaunchKernelGGL((valu_attn_kernel<T, D, NG, false, BATCH>), grid, block, 0, st, a, units, ngroups);
  return hipGetLastError();
}

template <typename T, int D, bool BATCH>
hipError_t launch_ng(const ValuArgs& a, dim3 grid, dim3 block, int NG, bool wgm, int64_t units, int ngroups,
                     hipStream_t st) {
  switch (NG) {
    case 1: return launch_one<T, D, 1, BATCH>(a, grid, block, wgm, units, ngroups, st);
    case 2: return launch_one<T, D, 2, BATCH>(a, grid, block, wgm, units, ngroups, st);
    case 4: return launch_one<T, D, 4, BATCH>(a, grid, block, wgm, units, ngroups, st);
    default: return launch_one<T, D, 8, BATCH>(a, grid, block, wgm, units, ngroups, st);
  }
}

template <typename T, int D>
hipError_t launch_typed(const ValuArgs& a, hipStream_t st) {
  const int G = a.s.Hq / a.s.Hkv;
  const int64_t N_b = (int64_t)a.s.R * a.s.B;
  int NG = (G >= 8) ? 8 : (G >= 4 ? 4 : (G >= 2 ? 2 : 1));
  if (G < 8 && (G & (G - 1))) NG = 8;  // non power of two: one masked group
  const int ngroups = (G + NG - 1) / NG;
  const int64_t units = N_b * a.s.Hkv * ngroups * a.splits;
  if (units == 0) return hipSuccess;
  // Splits written straight to the final output are merged in their workgroup.
  const bool wgm = a.splits > 1 && a.out.part_stride == 0;
  if (wgm && a.splits > kValuWgMax) return hipErrorInvalidValue;
  const int wpb = wgm ? a.splits : kValuWaves;
  const int64_t blocks = (units + wpb - 1) / wpb;
  dim3 grid((unsigned)blocks), block(wpb * 64);
  // bf16 waves that walk several batches (long generated tails) take the
  // batched updates; short runs (a few tokens per beam) the per-step ones,
  // which skip the steps that hold no key. Measured per Non-Shared pass:
  // batched, 512-token tails took 29.8 instead of 34.2 us, but 3-token tails
  // 19.7 instead of 16.7 us.
  if constexpr (sizeof(T) == 2) {
    if (a.chunk >= 64) return launch_ng<T, D, true>(a, grid, block, NG, wgm, units, ngroups, st);
  }
  return launch_ng<T, D, false>(a, grid, block, NG, wgm, units, ngroups, st);
}

}  // namespace

hipError_t launch_valu_attn(const ValuArgs& a, hipStream_t st) {
  if (a.dtype == 1) {
    return a.s.D == 64 ? launch_typed<uint16_t, 64>(a, st) : launch_typed<uint16_t, 128>(a, st);
  }
  return a.s.D == 64 ? launch_typed<float, 64>(a, st) : launch_typed<float, 128>(a, st);
}

}  // namespace xattn
