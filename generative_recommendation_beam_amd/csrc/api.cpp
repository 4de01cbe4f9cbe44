// C-ABI entry points: host-side validation, launch planning, workspace
// layout and dispatch. Nothing is enqueued unless every host-checkable
// argument is valid. These entry points never allocate, free or synchronize.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "xattn.h"
#include "kernels.h"

using namespace xattn;

namespace {

constexpr int kMaxBeamWidth = 16384;   // one request's table chunk must fit in LDS
constexpr int kTargetWaves = 2048;     // vector path: resident waves to cover 256 CUs
// MFMA path: split the prompt only until this many workgroups exist. Measured
// on MI355X, a split's partial write and in-kernel merge cost more than the
// extra parallelism returns once half the CUs hold a workgroup. When the
// generated tokens go to their own launch (long tails), the prompt splits
// join that launch's merge instead, and one workgroup per CU measured best
// (4096-token prompts, 512-token tails: 70.3 -> 67.1 us per call).
constexpr int kTargetMfmaBlocks = 128;
constexpr int kTargetMfmaBlocksLongTail = 256;
constexpr int kMinSplitKeys = 256;     // MFMA path: never split the prompt finer than this
// Vector path: a wave walks its keys a few rows per memory round trip, so a
// short prompt over few waves is latency-bound; splits down to this many keys
// (merged by one more launch) pay off there.
constexpr int kMinSplitKeysValu = 64;
constexpr int kValuWgMergeMax = 8;  // the vector kernel's in-workgroup split merge, at most
constexpr int kFuseMaxUnshared = 16;   // T_max up to this: Non-Shared part in the epilogue
// Generated tokens per Non-Shared split. Measured on MI355X with 512-token
// tails: 128 beats 64 (fewer partial rows to merge, half the wave starts).
constexpr int kUnsharedChunk = 128;
constexpr int kKeyGroupMinKeys = 512;  // automatic key groups only for prompts this long
constexpr int kNumCUs = 256;           // MI355X compute units

struct Plan {
  int mfma;
  int waves;
  int row_tiles;
  int p_splits;
  int p_chunk;
  int u_splits;  // 0 = fused into the prompt pass (or absent)
  int u_chunk;
  int parts;
  int ngroups;   // vector path: query-head groups per (beam, kv head)
  int stages;    // MFMA path: LDS pipeline stages
  int kgroups;   // MFMA path: wave groups taking alternate key tiles of the same rows
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// K/V buffers of an empty cache (no prompt tokens / no pool slots) may be NULL.
bool kv_ok(const void* k, const void* v, int64_t extent) {
  if (extent == 0) return (!k || aligned16(k)) && (!v || aligned16(v));
  return k && v && aligned16(k) && aligned16(v);
}

xattn_status check_dims(const xattn_dims* d) {
  if (!d) return XATTN_ERR_INVALID_ARG;
  if (d->num_requests < 0 || d->beam_width < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1)
    return XATTN_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return XATTN_ERR_INVALID_ARG;
  if (d->max_prefix_len < 0 || d->max_unshared_len < 1 || d->num_slots < 0 ||
      d->num_prefix_tokens < 0)
    return XATTN_ERR_INVALID_ARG;
  if (d->prefix_splits < 0 || d->unshared_splits < 0) return XATTN_ERR_INVALID_ARG;
  if (d->rows_per_block != 0 && d->rows_per_block != 32 && d->rows_per_block != 64 &&
      d->rows_per_block != 128)
    return XATTN_ERR_INVALID_ARG;
  if (d->pipeline_stages != 0 && d->pipeline_stages != 2 && d->pipeline_stages != 4)
    return XATTN_ERR_INVALID_ARG;
  if (d->key_groups < 0 || d->key_groups == 3 || d->key_groups > 4) return XATTN_ERR_INVALID_ARG;
  if (d->key_groups == 4 && d->pipeline_stages == 4) return XATTN_ERR_INVALID_ARG;  // LDS
  if (d->prompts_disjoint != 0 && d->prompts_disjoint != 1) return XATTN_ERR_INVALID_ARG;
  // The scale must be finite and positive: the kernels take a tile's running
  // maximum as max(q.k) * scale (a negative scale would make it the minimum)
  // and multiply masked scores of -inf by it (0 or inf would give NaN).
  // The kernels fold log2(e) into it, so that product must stay finite too.
  const float scale_log2 = d->scale * 1.4426950408889634f;
  if (!(d->scale > 0.0f && scale_log2 <= 3.4028234663852886e38f)) return XATTN_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return XATTN_ERR_UNSUPPORTED;
  if (d->key_groups == 4 && d->head_dim != 128) return XATTN_ERR_UNSUPPORTED;
  if (d->key_groups == 4 && d->rows_per_block == 128) return XATTN_ERR_UNSUPPORTED;  // 16 waves
  if (d->dtype != XATTN_F32 && d->dtype != XATTN_BF16) return XATTN_ERR_UNSUPPORTED;
  if (d->beam_width > kMaxBeamWidth) return XATTN_ERR_UNSUPPORTED;
  // Kernels address one (request, kv head) prompt with 32-bit byte offsets.
  const int64_t elem = d->dtype == XATTN_BF16 ? 2 : 4;
  if ((int64_t)d->max_prefix_len * d->head_dim * elem > (int64_t)INT32_MAX)
    return XATTN_ERR_UNSUPPORTED;
  const int64_t nb = (int64_t)d->num_requests * d->beam_width;
  if (nb * d->num_q_heads > (int64_t)INT32_MAX) return XATTN_ERR_UNSUPPORTED;
  return XATTN_OK;
}

// which: 0 shared stage, 1 unshared stage, 2 decode
Plan make_plan(const xattn_dims* d, int which) {
  Plan p{};
  p.kgroups = 1;
  const int G = d->num_q_heads / d->num_kv_heads;
  const int64_t M = (int64_t)d->beam_width * G;
  const int64_t N_b = (int64_t)d->num_requests * d->beam_width;
  const int maxP = d->max_prefix_len;
  const int T = d->max_unshared_len;
  // bf16 prompts always go to the matrix cores, even a single beam's few
  // query rows in a 32-row tile: measured on MI355X with 4 rows per (request,
  // kv head) and 4096-token prompts, the MFMA kernel streams the prompt
  // through LDS faster than the vector kernel walks it (237 against 273 us
  // per call with 64 distinct prompts, 163 against 232 us with 4 aliased).
  p.mfma = d->dtype == XATTN_BF16 ? 1 : 0;
  {
    const int NG = (G >= 8 || (G & (G - 1))) ? 8 : G;
    p.ngroups = (G + NG - 1) / NG;
  }
  const bool want_prefix = which != 1;
  const bool want_gen = which != 0;

  p.p_splits = 1;
  p.p_chunk = std::max(64, (int)cdiv(std::max(maxP, 1), 64) * 64);
  if (want_prefix) {
    int64_t base_units, target_units;
    if (p.mfma) {
      int rows = d->rows_per_block ? d->rows_per_block : (M >= 128 ? 128 : (M > 32 ? 64 : 32));
      int kg = d->key_groups ? d->key_groups : 1;
      if (d->key_groups == 0 && d->rows_per_block == 0 && d->pipeline_stages != 4 && M <= 32 &&
          d->head_dim == 128 && maxP >= kKeyGroupMinKeys)
        kg = 4;  // one row tile: four waves share its K/V tiles (aliased prompts: 163 -> 154 us)
      if (d->key_groups == 0 && d->rows_per_block == 0 && d->pipeline_stages != 4 && M >= 64 &&
          (int64_t)d->num_requests * d->num_kv_heads * cdiv(M, rows) < kNumCUs &&
          maxP >= kKeyGroupMinKeys) {
        // Too few (request, kv head, row tile) workgroups to cover the CUs:
        // take 64 rows per workgroup and split the keys of those rows over
        // wave groups, so twice the workgroups run and every wave walks a
        // share of the prompt. Head dim 128 takes four groups (two waves per
        // SIMD, which hides the loop's MFMA and LDS latency measured on
        // MI355X); other head dims take two.
        rows = 64;
        kg = d->head_dim == 128 ? 4 : 2;
      }
      p.kgroups = kg;
      p.waves = rows / 32 * kg;
      p.row_tiles = (int)cdiv(M, rows);
      base_units = (int64_t)d->num_requests * d->num_kv_heads * p.row_tiles;  // workgroups
      const bool long_tail = which == 2 && (d->unshared_splits > 0 || T > kFuseMaxUnshared);
      target_units = long_tail ? kTargetMfmaBlocksLongTail : kTargetMfmaBlocks;
    } else {
      p.waves = 1;
      p.row_tiles = 1;
      base_units = N_b * d->num_kv_heads * p.ngroups;  // wavefronts
      target_units = kTargetWaves;
    }
    int s;
    if (d->prefix_splits > 0) {
      s = d->prefix_splits;
    } else {
      s = base_units > 0 ? (int)cdiv(target_units, base_units) : 1;
      s = (int)std::min<int64_t>(s, std::max<int64_t>(1, cdiv(maxP, p.mfma ? kMinSplitKeys : kMinSplitKeysValu)));
      s = std::max(s, 1);
    }
    p.p_chunk = std::max(64, (int)cdiv(cdiv(std::max(maxP, 1), s), 64) * 64);
    p.p_splits = std::max(1, (int)cdiv(std::max(maxP, 1), p.p_chunk));
    if (d->prefix_splits > 0) p.p_splits = std::max(p.p_splits, 1);
  }
  p.u_splits = 0;
  p.u_chunk = T;
  if (want_gen) {
    if (which == 1) {
      // Non-Shared stage alone: split only long generated tails.
      const int s = d->unshared_splits > 0 ? d->unshared_splits
                                           : (T > 2 * kUnsharedChunk ? (int)cdiv(T, kUnsharedChunk) : 1);
      p.u_chunk = (int)cdiv(T, s);
      p.u_splits = (int)cdiv(T, p.u_chunk);
    } else {
      // decode: fuse into the prompt pass when short and not forced apart
      const bool fuse = d->unshared_splits == 0 && T <= kFuseMaxUnshared;
      if (!fuse) {
        const int s = d->unshared_splits > 0 ? d->unshared_splits : (int)cdiv(T, kUnsharedChunk);
        p.u_chunk = (int)cdiv(T, s);
        p.u_splits = (int)cdiv(T, p.u_chunk);
      }
    }
  }
  if (which == 0) p.parts = p.p_splits > 1 ? p.p_splits : 0;
  else if (which == 1) p.parts = p.u_splits > 1 ? p.u_splits : 0;
  else p.parts = (p.p_splits > 1 || p.u_splits > 0) ? p.p_splits + p.u_splits : 0;
  // A prompt split merged in-kernel with the Non-Shared tokens as its own
  // group member needs one more partial slot.
  if (which == 2 && p.mfma && p.p_splits > 1 && p.u_splits == 0) p.parts = p.p_splits + 1;
  // Vector path: a few prompt splits (and the short tail folded into split 0)
  // run as the waves of one workgroup and are merged there in LDS, so the
  // call needs no partials and no Merge launch.
  if (!p.mfma && which != 1 && p.p_splits > 1 && p.p_splits <= kValuWgMergeMax && p.u_splits == 0)
    p.parts = 0;
  // Two LDS stages measured best on every workload (four fit only one
  // workgroup per CU and push accumulators into AGPRs); four on request.
  p.stages = p.mfma ? (d->pipeline_stages ? d->pipeline_stages : 2) : 0;
  return p;
}

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace layout, the same for every call that needs one, so the counter
// block sits at the same place whatever call last used the buffer:
//   [counters: R*H_kv*row_tiles uint32, 256-aligned]   zero between calls
//   [partial O: parts * N_b*H_q * D float]
//   [partial lse: parts * N_b*H_q float]
struct Layout {
  size_t counters, o, lse, total;
};

// Does this plan merge prompt splits inside the MFMA kernel?
// (Partials are addressed with 32-bit byte offsets per split.)
bool uses_fixup(const xattn_dims* d, const Plan& p, int which) {
  const int64_t rows = (int64_t)d->num_requests * d->beam_width * d->num_q_heads;
  return p.mfma && p.p_splits > 1 && (which == 0 || (which == 2 && p.u_splits == 0)) &&
         rows * d->head_dim * 4 < (int64_t)INT32_MAX;
}

// Kernel launches one call makes under plan p.
// A decode's separate Non-Shared pass folds the prompt pass's partials into
// the final outputs (its splits merged in one workgroup): no Merge launch.
bool gen_folds_prompt(const Plan& p) { return p.u_splits > 0 && p.u_splits <= kValuWgMaxSplits; }

int launches(const xattn_dims* d, const Plan& p, int which) {
  if (p.parts == 0 || uses_fixup(d, p, which)) return 1;
  if (which == 2 && p.u_splits > 0) return gen_folds_prompt(p) ? 2 : 3;
  return 2;
}

// Does xattn_append_decode fold the append into a single decode launch
// under plan p? Its arrivals are counted per (request, kv head) over the row
// tiles, then per request over the kv heads.
bool append_folds(const xattn_dims* d, const Plan& p) {
  return p.mfma && p.parts == 0 && d->max_unshared_len < (1 << kArrivalShift) &&
         d->num_kv_heads <= kMaxAppendBlocks;
}

// With long generated tails (a Non-Shared pass of its own) the append folds
// into the MFMA prompt pass instead, done by prompt split 0's workgroups: the
// prompt pass reads neither the pool nor the tables, and the Non-Shared pass
// launched after it finds them updated. Its arrival counters are the head of
// the decode's counter block.
bool append_folds_prompt_pass(const xattn_dims* d, const Plan& p) {
  return p.mfma && p.parts > 0 && p.u_splits > 0 && !uses_fixup(d, p, 2) &&
         d->max_unshared_len < (1 << kArrivalShift) && d->num_kv_heads <= kMaxAppendBlocks;
}

// which = 3 (xattn_append_decode): the arrival counters of a folded append,
// else the decode's workspace.
Layout layout_for(const xattn_dims* d, const Plan& p, int which) {
  Layout L{0, 0, 0, 0};
  if (which == 3) {
    if (append_folds(d, p)) {
      L.total = align256((size_t)d->num_requests * d->num_kv_heads * sizeof(unsigned));
      return L;
    }
    which = 2;
  }
  const int64_t rows = (int64_t)d->num_requests * d->beam_width * d->num_q_heads;
  const int parts = p.parts;
  if (parts == 0) return L;
  const size_t nctr = (size_t)d->num_requests * d->num_kv_heads * std::max(p.row_tiles, 1);
  L.counters = 0;
  L.o = align256(nctr * sizeof(unsigned));
  L.lse = L.o + align256((size_t)parts * rows * d->head_dim * sizeof(float));
  L.total = L.lse + align256((size_t)parts * rows * sizeof(float));
  return L;
}

size_t ws_bytes_for(const xattn_dims* d, const Plan& p, int which) {
  return layout_for(d, p, which).total;
}

Shape make_shape(const xattn_dims* d) {
  Shape s;
  s.R = d->num_requests;
  s.B = d->beam_width;
  s.Hq = d->num_q_heads;
  s.Hkv = d->num_kv_heads;
  s.D = d->head_dim;
  s.T_max = d->max_unshared_len;
  s.n_ptok = d->num_prefix_tokens;
  s.scale_log2 = d->scale * 1.4426950408889634f;
  return s;
}

struct Workspace {
  unsigned* counters;
  float* o;
  float* lse;
};

Workspace carve(const xattn_dims* d, const Plan& p, int which, void* ws) {
  const Layout L = layout_for(d, p, which);
  char* base = static_cast<char*>(ws);
  return Workspace{reinterpret_cast<unsigned*>(base + L.counters),
                   reinterpret_cast<float*>(base + L.o), reinterpret_cast<float*>(base + L.lse)};
}

inline xattn_status hip_status(hipError_t e) { return e == hipSuccess ? XATTN_OK : XATTN_ERR_HIP; }

// Launch the prompt pass (MFMA or vector). `mode` selects how the MFMA kernel
// writes (final / partial slot part_base+split / in-kernel split merge).
// kp != null folds the Non-Shared tokens into prompt split 0.
// The cache append folded into a single-launch decode (see xattn_append_decode).
struct FusedAppend {
  const void* k_new;
  const void* v_new;
  const int32_t* parent;
  const int64_t* slot_base;
  const uint8_t* active;
  void* k_pool;
  void* v_pool;
  int32_t* table_out;
  int32_t* ulen;
};

hipError_t run_prefix(const xattn_dims* d, const Plan& p, int mode, const void* q, const void* ks,
                      const void* vs, const int64_t* poff, const int32_t* plen, const void* kp,
                      const void* vp, const int32_t* table, const int32_t* ulen, OutSpec out,
                      const Workspace& w, hipStream_t st, const FusedAppend* fa = nullptr) {
  const int64_t rows = (int64_t)d->num_requests * d->beam_width * d->num_q_heads;
  if (p.mfma) {
    SharedMfmaArgs a;
    a.s = make_shape(d);
    a.q = static_cast<const uint16_t*>(q);
    a.k_shared = static_cast<const uint16_t*>(ks);
    a.v_shared = static_cast<const uint16_t*>(vs);
    a.prefix_off = poff;
    a.prefix_len = plen;
    a.k_pool = static_cast<const uint16_t*>(kp);
    a.v_pool = static_cast<const uint16_t*>(vp);
    a.slot_table = table;
    a.unshared_len = ulen;
    a.out = out;
    a.mode = mode;
    a.part_o = w.o;
    a.part_lse = w.lse;
    a.part_stride = rows;
    a.counters = w.counters;
    a.waves = p.waves;
    a.row_tiles = p.row_tiles;
    a.p_splits = p.p_splits;
    a.p_chunk = p.p_chunk;
    a.gen_member = (mode == kModeFixup && kp != nullptr) ? 1 : 0;
    a.stages = p.stages;
    a.key_groups = p.kgroups;
    // A workgroup alone reads its prompt keys: one row tile, and no other
    // request's prompt overlaps (the caller's guarantee).
    a.stream_kv = d->prompts_disjoint != 0 && p.row_tiles == 1;
    a.append = fa ? 1 : 0;
    a.k_new = fa ? static_cast<const uint16_t*>(fa->k_new) : nullptr;
    a.v_new = fa ? static_cast<const uint16_t*>(fa->v_new) : nullptr;
    a.parent = fa ? fa->parent : nullptr;
    a.slot_base = fa ? fa->slot_base : nullptr;
    a.active = fa ? fa->active : nullptr;
    a.k_pool_out = fa ? static_cast<uint16_t*>(fa->k_pool) : nullptr;
    a.v_pool_out = fa ? static_cast<uint16_t*>(fa->v_pool) : nullptr;
    a.table_out = fa ? fa->table_out : nullptr;
    a.ulen_rw = fa ? fa->ulen : nullptr;
    a.arrivals = d->num_kv_heads;  // per request, after each (request, kv head) has counted its row tiles
    {
      const int64_t row_bytes = (int64_t)d->num_kv_heads * d->head_dim * 2;
      const int64_t new_rows = (int64_t)d->num_requests * d->beam_width;
      const bool small_pool = (int64_t)d->num_slots * row_bytes < (int64_t(1) << 32) &&
                              (!fa || new_rows * row_bytes < (int64_t(1) << 32));
      a.token_block = kp != nullptr && small_pool && d->num_q_heads == 4 * d->num_kv_heads &&
                      d->max_unshared_len <= 3 && d->head_dim == 128;
      a.pool_bytes = small_pool ? (uint32_t)((int64_t)d->num_slots * row_bytes) : 0u;
      a.new_bytes = (small_pool && fa) ? (uint32_t)(new_rows * row_bytes) : 0u;
    }
    return launch_shared_mfma(a, st);
  }
  ValuArgs a{};
  a.s = make_shape(d);
  a.dtype = d->dtype;
  a.q = q;
  a.k_shared = ks;
  a.v_shared = vs;
  a.prefix_off = poff;
  a.prefix_len = plen;
  a.k_pool = kp;
  a.v_pool = vp;
  a.slot_table = table;
  a.unshared_len = ulen;
  a.use_prefix = 1;
  a.use_gen = kp != nullptr ? 1 : 0;
  a.splits = p.p_splits;
  a.chunk = p.p_chunk;
  a.out = mode == kModeFinal ? out : OutSpec{w.o, w.lse, rows, out.part_base};
  return launch_valu_attn(a, st);
}

// fold: the prompt pass's partial slots (workspace) folded into final
// outputs by this launch (no Merge launch); null: `out` as given.
hipError_t run_gen(const xattn_dims* d, const Plan& p, const void* q, const void* kp,
                   const void* vp, const int32_t* table, const int32_t* ulen, OutSpec out,
                   hipStream_t st, const Workspace* fold = nullptr) {
  ValuArgs a{};
  a.s = make_shape(d);
  a.dtype = d->dtype;
  a.q = q;
  a.k_shared = nullptr;
  a.v_shared = nullptr;
  a.prefix_off = nullptr;
  a.prefix_len = nullptr;
  a.k_pool = kp;
  a.v_pool = vp;
  a.slot_table = table;
  a.unshared_len = ulen;
  a.use_prefix = 0;
  a.use_gen = 1;
  a.splits = std::max(1, p.u_splits);
  a.chunk = p.u_chunk;
  a.out = out;
  if (fold) {
    a.fold_o = fold->o;
    a.fold_lse = fold->lse;
    a.fold_parts = p.p_splits;
    a.fold_stride = (int64_t)d->num_requests * d->beam_width * d->num_q_heads;
  }
  return launch_valu_attn(a, st);
}



}  // namespace

extern "C" {

const char* xattn_status_string(xattn_status s) {
  switch (s) {
    case XATTN_OK: return "XATTN_OK";
    case XATTN_ERR_INVALID_ARG: return "XATTN_ERR_INVALID_ARG: invalid argument";
    case XATTN_ERR_UNSUPPORTED: return "XATTN_ERR_UNSUPPORTED: shape or dtype not supported";
    case XATTN_ERR_WORKSPACE: return "XATTN_ERR_WORKSPACE: workspace missing or too small";
    case XATTN_ERR_HIP: return "XATTN_ERR_HIP: HIP launch error";
  }
  return "XATTN_UNKNOWN_STATUS";
}

xattn_status xattn_get_plan(const xattn_dims* d, int which, xattn_plan* out) {
  xattn_status e = check_dims(d);
  if (e != XATTN_OK) return e;
  if (!out || which < 0 || which > 2) return XATTN_ERR_INVALID_ARG;
  const Plan p = make_plan(d, which);
  out->rows_per_block = p.mfma ? 32 * p.waves / p.kgroups : 0;
  out->row_tiles = p.mfma ? p.row_tiles : 0;
  out->prefix_splits = which == 1 ? 0 : p.p_splits;
  out->prefix_chunk = which == 1 ? 0 : p.p_chunk;
  out->unshared_splits = p.u_splits;
  out->unshared_chunk = which == 0 ? 0 : p.u_chunk;
  out->partials = p.parts;
  out->mfma = p.mfma;
  out->launches = launches(d, p, which);
  out->pipeline_stages = p.stages;
  out->key_groups = p.mfma ? p.kgroups : 0;
  return XATTN_OK;
}

xattn_status xattn_workspace_size(const xattn_dims* d, int which, size_t* bytes) {
  xattn_status e = check_dims(d);
  if (e != XATTN_OK) return e;
  if (!bytes || which < 0 || which > 3) return XATTN_ERR_INVALID_ARG;
  *bytes = ws_bytes_for(d, make_plan(d, which == 3 ? 2 : which), which);
  return XATTN_OK;
}

xattn_status xattn_shared_stage(const xattn_dims* d, const void* q, const void* ks, const void* vs,
                                const int64_t* poff, const int32_t* plen, float* o, float* lse,
                                void* ws, size_t ws_bytes, void* stream) {
  xattn_status e = check_dims(d);
  if (e != XATTN_OK) return e;
  if (!q || !poff || !plen || !o || !lse) return XATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(o) || !kv_ok(ks, vs, d->num_prefix_tokens))
    return XATTN_ERR_INVALID_ARG;
  const Plan p = make_plan(d, 0);
  const size_t need = ws_bytes_for(d, p, 0);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return XATTN_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t rows = (int64_t)d->num_requests * d->beam_width * d->num_q_heads;
  const Workspace w = need > 0 ? carve(d, p, 0, ws) : Workspace{nullptr, nullptr, nullptr};
  const OutSpec fin{o, lse, 0, 0};
  if (p.parts == 0)
    return hip_status(run_prefix(d, p, kModeFinal, q, ks, vs, poff, plen, nullptr, nullptr, nullptr,
                                 nullptr, fin, w, st));
  if (uses_fixup(d, p, 0))
    return hip_status(run_prefix(d, p, kModeFixup, q, ks, vs, poff, plen, nullptr, nullptr, nullptr,
                                 nullptr, fin, w, st));
  hipError_t he = run_prefix(d, p, kModePartial, q, ks, vs, poff, plen, nullptr, nullptr, nullptr,
                             nullptr, fin, w, st);
  if (he != hipSuccess) return XATTN_ERR_HIP;
  return hip_status(launch_merge_parts(rows, d->head_dim, p.parts, w.o, w.lse, o, lse, st));
}

xattn_status xattn_unshared_stage(const xattn_dims* d, const void* q, const void* kp,
                                  const void* vp, const int32_t* table, const int32_t* ulen,
                                  float* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  xattn_status e = check_dims(d);
  if (e != XATTN_OK) return e;
  if (!q || !table || !ulen || !o || !lse) return XATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(o) || !kv_ok(kp, vp, d->num_slots)) return XATTN_ERR_INVALID_ARG;
  const Plan p = make_plan(d, 1);
  const size_t need = ws_bytes_for(d, p, 1);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return XATTN_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t rows = (int64_t)d->num_requests * d->beam_width * d->num_q_heads;
  if (p.parts == 0) {
    Plan p1 = p;
    p1.u_splits = 1;
    return hip_status(run_gen(d, p1, q, kp, vp, table, ulen, OutSpec{o, lse, 0, 0}, st));
  }
  const Workspace w = carve(d, p, 1, ws);
  hipError_t he = run_gen(d, p, q, kp, vp, table, ulen, OutSpec{w.o, w.lse, rows, 0}, st);
  if (he != hipSuccess) return XATTN_ERR_HIP;
  return hip_status(launch_merge_parts(rows, d->head_dim, p.parts, w.o, w.lse, o, lse, st));
}

xattn_status xattn_merge(int64_t rows, int32_t head_dim, const float* o_a, const float* lse_a,
                         const float* o_b, const float* lse_b, float* o_out, float* lse_out,
                         void* stream) {
  if (rows < 0 || head_dim <= 0) return XATTN_ERR_INVALID_ARG;
  // a row's threads (head_dim / 4 of them) must tile a 256-thread block
  if (head_dim % 4 != 0 || 256 % (head_dim / 4) != 0) return XATTN_ERR_UNSUPPORTED;
  if (rows == 0) return XATTN_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out) return XATTN_ERR_INVALID_ARG;
  if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o_out)) return XATTN_ERR_INVALID_ARG;
  return hip_status(launch_merge2(rows, head_dim, o_a, lse_a, o_b, lse_b, o_out, lse_out,
                                  static_cast<hipStream_t>(stream)));
}

xattn_status xattn_decode(const xattn_dims* d, const void* q, const void* ks, const void* vs,
                          const int64_t* poff, const int32_t* plen, const void* kp, const void* vp,
                          const int32_t* table, const int32_t* ulen, float* o, float* lse,
                          void* ws, size_t ws_bytes, void* stream) {
  xattn_status e = check_dims(d);
  if (e != XATTN_OK) return e;
  if (!q || !poff || !plen || !table || !ulen || !o) return XATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(o) || !kv_ok(ks, vs, d->num_prefix_tokens) ||
      !kv_ok(kp, vp, d->num_slots))
    return XATTN_ERR_INVALID_ARG;
  const Plan p = make_plan(d, 2);
  const size_t need = ws_bytes_for(d, p, 2);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return XATTN_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t rows = (int64_t)d->num_requests * d->beam_width * d->num_q_heads;
  const Workspace w = need > 0 ? carve(d, p, 2, ws) : Workspace{nullptr, nullptr, nullptr};
  const OutSpec fin{o, lse, 0, 0};
  if (p.parts == 0)  // one launch: prompt pass with the Non-Shared tokens folded in
    return hip_status(run_prefix(d, p, kModeFinal, q, ks, vs, poff, plen, kp, vp, table, ulen,
                                 fin, w, st));
  if (uses_fixup(d, p, 2))  // one launch: prompt splits merged by their last workgroup
    return hip_status(run_prefix(d, p, kModeFixup, q, ks, vs, poff, plen, kp, vp, table, ulen,
                                 fin, w, st));
  const bool fused = p.u_splits == 0;
  hipError_t he = run_prefix(d, p, kModePartial, q, ks, vs, poff, plen, fused ? kp : nullptr,
                             fused ? vp : nullptr, table, ulen, fin, w, st);
  if (he != hipSuccess) return XATTN_ERR_HIP;
  if (!fused) {
    if (gen_folds_prompt(p))  // the Non-Shared pass merges everything into o/lse
      return hip_status(run_gen(d, p, q, kp, vp, table, ulen, fin, st, &w));
    he = run_gen(d, p, q, kp, vp, table, ulen, OutSpec{w.o, w.lse, rows, p.p_splits}, st);
    if (he != hipSuccess) return XATTN_ERR_HIP;
  }
  return hip_status(launch_merge_parts(rows, d->head_dim, p.parts, w.o, w.lse, o, lse, st));
}

xattn_status xattn_cache_append(const xattn_dims* d, const void* k_new, const void* v_new,
                                const int32_t* parent, const int64_t* slot_base,
                                const uint8_t* active, void* k_pool, void* v_pool,
                                const int32_t* table_in, int32_t* table_out, int32_t* ulen,
                                void* stream) {
  xattn_status e = check_dims(d);
  if (e != XATTN_OK) return e;
  if (!k_new || !v_new || !parent || !slot_base || !k_pool || !v_pool || !table_in ||
      !table_out || !ulen)
    return XATTN_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return XATTN_ERR_INVALID_ARG;
  const int64_t N_b = (int64_t)d->num_requests * d->beam_width;
  if (d->num_requests > 0 && d->num_slots < N_b) return XATTN_ERR_INVALID_ARG;
  AppendArgs a;
  a.R = d->num_requests;
  a.B = d->beam_width;
  a.Hkv = d->num_kv_heads;
  a.D = d->head_dim;
  a.T_max = d->max_unshared_len;
  a.elem_bytes = d->dtype == XATTN_BF16 ? 2 : 4;
  a.k_new = k_new;
  a.v_new = v_new;
  a.parent = parent;
  a.slot_base = slot_base;
  a.active = active;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.table_in = table_in;
  a.table_out = table_out;
  a.unshared_len = ulen;
  if (!append_supported(a)) return XATTN_ERR_UNSUPPORTED;
  return hip_status(launch_append(a, static_cast<hipStream_t>(stream)));
}

xattn_status xattn_append_decode(const xattn_dims* d, const void* q, const void* ks, const void* vs,
                                 const int64_t* poff, const int32_t* plen, const void* k_new,
                                 const void* v_new, const int32_t* parent, const int64_t* slot_base,
                                 const uint8_t* active, void* kp, void* vp, const int32_t* table_in,
                                 int32_t* table_out, int32_t* ulen, float* o, float* lse, void* ws,
                                 size_t ws_bytes, void* stream) {
  xattn_status e = check_dims(d);
  if (e != XATTN_OK) return e;
  if (!q || !poff || !plen || !k_new || !v_new || !parent || !slot_base || !kp || !vp || !table_in ||
      !table_out || !ulen || !o)
    return XATTN_ERR_INVALID_ARG;
  if (table_in == table_out) return XATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(o) || !aligned16(k_new) || !aligned16(v_new) ||
      !kv_ok(ks, vs, d->num_prefix_tokens) || !kv_ok(kp, vp, d->num_slots))
    return XATTN_ERR_INVALID_ARG;
  const int64_t N_b = (int64_t)d->num_requests * d->beam_width;
  if (d->num_requests > 0 && d->num_slots < N_b) return XATTN_ERR_INVALID_ARG;
  const Plan p = make_plan(d, 2);
  const size_t need = ws_bytes_for(d, p, 3);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return XATTN_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (append_folds_prompt_pass(d, p)) {
    if (d->num_requests == 0) return XATTN_OK;
    const int64_t rows = (int64_t)d->num_requests * d->beam_width * d->num_q_heads;
    const Workspace w = carve(d, p, 2, ws);
    const FusedAppend fa{k_new, v_new, parent, slot_base, active, kp, vp, table_out, ulen};
    if (run_prefix(d, p, kModePartial, q, ks, vs, poff, plen, nullptr, nullptr, table_in, ulen,
                   OutSpec{o, lse, 0, 0}, w, st, &fa) != hipSuccess)
      return XATTN_ERR_HIP;
    if (gen_folds_prompt(p))  // the Non-Shared pass merges everything into o/lse
      return hip_status(run_gen(d, p, q, kp, vp, table_out, ulen, OutSpec{o, lse, 0, 0}, st, &w));
    if (run_gen(d, p, q, kp, vp, table_out, ulen, OutSpec{w.o, w.lse, rows, p.p_splits}, st) != hipSuccess)
      return XATTN_ERR_HIP;
    return hip_status(launch_merge_parts(rows, d->head_dim, p.parts, w.o, w.lse, o, lse, st));
  }
  if (!append_folds(d, p)) {
    e = xattn_cache_append(d, k_new, v_new, parent, slot_base, active, kp, vp, table_in, table_out,
                           ulen, stream);
    if (e != XATTN_OK) return e;
    return xattn_decode(d, q, ks, vs, poff, plen, kp, vp, table_out, ulen, o, lse, ws, ws_bytes, stream);
  }
  if (d->num_requests == 0) return XATTN_OK;
  const FusedAppend fa{k_new, v_new, parent, slot_base, active, kp, vp, table_out, ulen};
  const Workspace w{static_cast<unsigned*>(ws), nullptr, nullptr};
  return hip_status(run_prefix(d, p, kModeFinal, q, ks, vs, poff, plen, kp, vp, table_in, ulen,
                               OutSpec{o, lse, 0, 0}, w, st, &fa));
}

}  // extern "C"

// ---- xattn_append_decode_static: the workspace in a device-resident array ----
namespace {

// The largest workspace the allocation-free entry point serves: the folded
// append needs R*H_kv counters; unfolded plans (long generated tails, split
// prompts) also need their partial outputs.
constexpr size_t kStaticWorkspaceBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

// One copy per GPU, alive until the process ends. In host code this name is
// only a handle for hipGetSymbolAddress: kernels and copies take the device
// address it returns (static_ws_ptr[dev]).
__device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

void* static_ws_ptr[kMaxDevices];
hipError_t static_ws_err[kMaxDevices];
std::once_flag static_ws_once[kMaxDevices];

__global__ __launch_bounds__(256) void zero_words_kernel(unsigned* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

}  // namespace

extern "C" {

xattn_status xattn_append_decode_static(const xattn_dims* d, const void* q, const void* ks, const void* vs,
                                        const int64_t* poff, const int32_t* plen, const void* k_new,
                                        const void* v_new, const int32_t* parent, const int64_t* slot_base,
                                        const uint8_t* active, void* kp, void* vp, const int32_t* table_in,
                                        int32_t* table_out, int32_t* ulen, float* o, float* lse, void* stream) {
  xattn_status e = check_dims(d);
  if (e != XATTN_OK) return e;
  const Plan p = make_plan(d, 2);
  const Layout L = layout_for(d, p, 3);
  if (L.total > kStaticWorkspaceBytes) return XATTN_ERR_WORKSPACE;  // beyond the fixed array
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return XATTN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return XATTN_ERR_UNSUPPORTED;
  std::call_once(static_ws_once[dev], [dev] {
    static_ws_err[dev] = hipGetSymbolAddress(&static_ws_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (static_ws_err[dev] != hipSuccess || static_ws_ptr[dev] == nullptr) return XATTN_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // The split counters at the head of the workspace must be zero; the array
  // keeps whatever the last call left, so they are cleared here (a fill
  // kernel, not a memset node, so that a captured graph replays it cleanly).
  const size_t ctr_bytes = L.o > 0 ? L.o : L.total;
  if (ctr_bytes > 0) {
    const int64_t words = (int64_t)(ctr_bytes / 4);
    const unsigned grid = (unsigned)std::min<int64_t>(std::max<int64_t>((words + 255) / 256, 1), 1024);
    hipLaunchKernelGGL(zero_words_kernel, dim3(grid), dim3(256), 0, st, static_cast<unsigned*>(static_ws_ptr[dev]),
                       words);
    if (hipGetLastError() != hipSuccess) return XATTN_ERR_HIP;
  }
  return xattn_append_decode(d, q, ks, vs, poff, plen, k_new, v_new, parent, slot_base, active, kp, vp, table_in,
                             table_out, ulen, o, lse, static_ws_ptr[dev], L.total, stream);
}

static size_t paged_ws_bytes(const xattn_dims* d, int32_t max_seq_len) {
  const int nparts = max_seq_len > kPagedPart ? (max_seq_len + kPagedPart - 1) / kPagedPart : 1;
  if (nparts <= 1) return 0;
  const int64_t rows = (int64_t)d->num_requests * d->beam_width * d->num_q_heads;
  return align256((size_t)nparts * rows * d->head_dim * sizeof(float)) +
         align256((size_t)nparts * rows * sizeof(float));
}

static xattn_status paged_check(const xattn_dims* d, int32_t max_seq_len) {
  xattn_status e = check_dims(d);
  if (e != XATTN_OK) return e;
  if (max_seq_len < 0) return XATTN_ERR_INVALID_ARG;
  if (d->dtype != XATTN_BF16) return XATTN_ERR_UNSUPPORTED;
  return XATTN_OK;
}

xattn_status xattn_paged_workspace_size(const xattn_dims* d, int32_t max_seq_len, size_t* bytes) {
  xattn_status e = paged_check(d, max_seq_len);
  if (e != XATTN_OK) return e;
  if (!bytes) return XATTN_ERR_INVALID_ARG;
  *bytes = paged_ws_bytes(d, max_seq_len);
  return XATTN_OK;
}

xattn_status xattn_paged_decode(const xattn_dims* d, int32_t max_seq_len, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_table, int32_t max_blocks,
                                const int32_t* seq_len, float* o, float* lse, void* ws, size_t ws_bytes,
                                void* stream) {
  xattn_status e = paged_check(d, max_seq_len);
  if (e != XATTN_OK) return e;
  if (!q || !k_cache || !v_cache || !block_table || !seq_len || !o) return XATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return XATTN_ERR_INVALID_ARG;
  if (max_blocks < 0 || (int64_t)max_blocks * kPagedBlock < max_seq_len) return XATTN_ERR_INVALID_ARG;
  const size_t need = paged_ws_bytes(d, max_seq_len);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return XATTN_ERR_WORKSPACE;
  PagedArgs a;
  a.Hq = d->num_q_heads;
  a.Hkv = d->num_kv_heads;
  a.D = d->head_dim;
  a.max_blocks = max_blocks;
  a.nparts = max_seq_len > kPagedPart ? (max_seq_len + kPagedPart - 1) / kPagedPart : 1;
  a.rows = (int64_t)d->num_requests * d->beam_width * d->num_q_heads;
  a.scale_log2 = d->scale * 1.4426950408889634f;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.block_table = block_table;
  a.seq_len = seq_len;
  a.o = o;
  a.lse = lse;
  char* base = static_cast<char*>(ws);
  a.part_o = need ? reinterpret_cast<float*>(base) : nullptr;
  a.part_lse = need ? reinterpret_cast<float*>(base + align256((size_t)a.nparts * a.rows * a.D * sizeof(float)))
                    : nullptr;
  return hip_status(launch_paged_attn(a, static_cast<hipStream_t>(stream)));
}

xattn_status xattn_paged_copy_blocks(const xattn_dims* d, void* k_cache, void* v_cache, const int32_t* src,
                                     const int32_t* dst, int32_t n, void* stream) {
  xattn_status e = paged_check(d, 0);
  if (e != XATTN_OK) return e;
  if (n < 0) return XATTN_ERR_INVALID_ARG;
  if (n == 0) return XATTN_OK;
  if (!k_cache || !v_cache || !src || !dst || !aligned16(k_cache) || !aligned16(v_cache))
    return XATTN_ERR_INVALID_ARG;
  const int64_t block_elems = (int64_t)d->num_kv_heads * kPagedBlock * d->head_dim;
  return hip_status(launch_copy_blocks(static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), src,
                                       dst, n, block_elems, static_cast<hipStream_t>(stream)));
}

xattn_status xattn_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return XATTN_OK;
  if (!src || !sink || !aligned16(src) || bytes % 16 != 0) return XATTN_ERR_INVALID_ARG;
  return hip_status(launch_stream_read(src, (int64_t)bytes, sink, static_cast<hipStream_t>(stream)));
}

xattn_status xattn_beam_topk(int32_t num_requests, int32_t beam_width, int32_t top_k, int32_t n_out,
                             const float* beam_score, const float* logprob, const int32_t* token,
                             int32_t* parent, int32_t* token_out, float* score_out, void* stream) {
  if (num_requests < 0 || beam_width < 1 || top_k < 1 || n_out < 0) return XATTN_ERR_INVALID_ARG;
  if ((int64_t)beam_width * top_k < n_out) return XATTN_ERR_INVALID_ARG;
  if (num_requests == 0 || n_out == 0) return XATTN_OK;
  if (!beam_score || !logprob || !token || !parent || !token_out || !score_out)
    return XATTN_ERR_INVALID_ARG;
  if (beam_width > kTopkMaxBeams || n_out > kTopkMaxOut || top_k > kTopkCap - n_out)
    return XATTN_ERR_UNSUPPORTED;
  TopkArgs a;
  a.R = num_requests;
  a.BW = beam_width;
  a.K = top_k;
  a.n_out = n_out;
  a.beam_score = beam_score;
  a.logprob = logprob;
  a.token = token;
  a.parent = parent;
  a.token_out = token_out;
  a.score_out = score_out;
  return hip_status(launch_beam_topk(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
