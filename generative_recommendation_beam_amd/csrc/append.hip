// Token-granular Non-Shared cache append (xGR page, section 2.1 xAttention:
// token-level management of the Non-Shared cache and in-place updates through
// direct indices without read-before-write hazards).
//
// Slot-table column j of a new beam depends only on column j of its parent's
// row, so the table update splits into independent column chunks. One
// workgroup owns one (request, column chunk): it reads the chunk of every
// parent row of the request into LDS, waits at a barrier, then writes the new
// rows. No other workgroup touches those table cells, so table_out may alias
// table_in. Further workgroups of the same launch copy the new K/V rows into
// their pool slots.
//
// Every workgroup of request r needs t = unshared_len[r] before it is
// incremented, and only one launch is made: each workgroup adds one arrival
// in the bits above kArrivalShift of unshared_len[r] with an atomic that also
// returns t (the low bits), and the last arrival stores the new length (t + 1,
// or t for an inactive request or a full row). Nothing else reads
// unshared_len during the launch.
//
// A workgroup requests everything that does not depend on t (its K/V pieces,
// or its table chunk's cells of every row and the parent of each cell's row,
// with indices clamped rather than branched on) before the arrival, so the
// loads, the atomic and the activity flag are in flight together and the
// stores follow one round trip after the start.
#include "device.h"
#include "kernels.h"

namespace xattn {

namespace {

constexpr int kAppendThreads = 256;
constexpr int kCells = 8;   // table cells per thread held in registers across the arrival
constexpr int kPieces = 2;  // 16-byte K (and V) pieces per thread held across the arrival

struct AppendPlan {
  int col_chunk;   // table columns per workgroup
  int col_blocks;  // workgroups per request for the table
  int kv_blocks;   // workgroups per request for the K/V copy
};

AppendPlan plan_append(const AppendArgs& a) {
  AppendPlan p;
  p.col_chunk = kAppendThreads * kCells / a.B;
  if (p.col_chunk < 1) p.col_chunk = 1;
  if (p.col_chunk > a.T_max) p.col_chunk = a.T_max;
  p.col_blocks = (a.T_max + p.col_chunk - 1) / p.col_chunk;
  const int64_t pieces = (int64_t)a.B * a.Hkv * a.D * a.elem_bytes / 16;
  const int64_t kv = (pieces + kAppendThreads * kPieces - 1) / (kAppendThreads * kPieces);
  p.kv_blocks = (int)(kv < 1 ? 1 : (kv > kMaxAppendBlocks / 2 ? kMaxAppendBlocks / 2 : kv));
  return p;
}

// Arrive at request r's counter. Wave 0 makes the atomic while wave 1 reads
// the request's activity flag and slot base, beside the workgroup's own
// loads. Returns this call's position t to every thread, whether the request
// takes a new token (active, row not full), and the slot base; the last of
// the request's nblk workgroups stores the new length.
struct Arrival {
  int t;
  bool grow;
  int64_t sbase;
};
__device__ __forceinline__ Arrival arrive(int32_t* ulen, const uint8_t* active, const int64_t* slot_base, int r,
                                          int nblk, int T_max) {
  __shared__ int s_old, s_on;
  __shared__ int64_t s_sb;
  if (threadIdx.x == 0) s_old = atomicAdd(ulen + r, 1 << kArrivalShift);
  if (threadIdx.x == 64) {
    s_on = active ? active[r] : 1;
    s_sb = slot_base[r];
  }
  __syncthreads();
  const int old = s_old;
  const int t = old & ((1 << kArrivalShift) - 1);
  const bool grow = s_on != 0 && t < T_max;
  if (threadIdx.x == 0 && (old >> kArrivalShift) == nblk - 1) ulen[r] = grow ? t + 1 : t;
  return Arrival{t, grow, s_sb};
}

__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a, AppendPlan p) {
  extern __shared__ int32_t staged[];  // [B][col_chunk]
  const int r = blockIdx.x;
  const int y = blockIdx.y;
  const int nblk = p.col_blocks + p.kv_blocks;
  const int B = a.B;
  const int64_t nbase = (int64_t)r * B;
  const int tid = threadIdx.x;

  if (y < p.col_blocks) {
    // Columns [c0, c0 + cw) of every row of request r. Cell i is (row i / cw,
    // column c0 + i % cw); columns at or past t are read but not used.
    const int c0 = y * p.col_chunk;
    const int cw = min(p.col_chunk, a.T_max - c0);
    const int cells = B * cw;
    const int32_t* tin = a.table_in + nbase * a.T_max + c0;
    int32_t val[kCells], par[kCells];
#pragma unroll
    for (int k = 0; k < kCells; ++k) {
      const int ic = min(tid + k * kAppendThreads, cells - 1);
      const int b = ic / cw;
      val[k] = tin[(int64_t)b * a.T_max + (ic - b * cw)];
      par[k] = a.parent[nbase + b];
    }
    const Arrival av = arrive(a.unshared_len, a.active, a.slot_base, r, nblk, a.T_max);
    const int t = av.t;
    // A request that takes no token keeps its rows: copied into a separate
    // table_out (nothing to do in place).
    if (!av.grow) {
      if (a.table_out == a.table_in) return;
      int32_t* tout = a.table_out + nbase * a.T_max + c0;
      for (int i = tid; i < cells; i += kAppendThreads) {
        const int b = i / cw, c = i - b * cw;
        if (c0 + c < t) tout[(int64_t)b * a.T_max + c] = tin[(int64_t)b * a.T_max + c];
      }
      return;
    }
    if (c0 < t) {
#pragma unroll
      for (int k = 0; k < kCells; ++k) {
        const int i = tid + k * kAppendThreads;
        if (i < cells) {
          const int b = i / cw;
          staged[b * p.col_chunk + (i - b * cw)] = val[k];
        }
      }
      for (int i = tid + kCells * kAppendThreads; i < cells; i += kAppendThreads) {  // beam widths above 2048
        const int b = i / cw;
        staged[b * p.col_chunk + (i - b * cw)] = tin[(int64_t)b * a.T_max + (i - b * cw)];
      }
      __syncthreads();
      int32_t* tout = a.table_out + nbase * a.T_max + c0;
#pragma unroll
      for (int k = 0; k < kCells; ++k) {
        const int i = tid + k * kAppendThreads;
        const int b = i / cw, c = i - b * cw;
        if (i < cells && c0 + c < t) tout[(int64_t)b * a.T_max + c] = staged[par[k] * p.col_chunk + c];
      }
      for (int i = tid + kCells * kAppendThreads; i < cells; i += kAppendThreads) {
        const int b = i / cw, c = i - b * cw;
        if (c0 + c < t) tout[(int64_t)b * a.T_max + c] = staged[a.parent[nbase + b] * p.col_chunk + c];
      }
    }
    if (y == 0) {
      const int64_t sb = av.sbase + (int64_t)t * B;
      for (int b = tid; b < B; b += kAppendThreads) a.table_out[(nbase + b) * a.T_max + t] = (int32_t)(sb + b);
    }
    return;
  }

  // K/V copy: 16-byte pieces of the request's [B][H_kv][D] rows.
  const int64_t row_bytes = (int64_t)a.Hkv * a.D * a.elem_bytes;
  const int64_t total = row_bytes / 16 * B;
  const int64_t stride = (int64_t)p.kv_blocks * kAppendThreads;
  const int64_t i0 = (int64_t)(y - p.col_blocks) * kAppendThreads + tid;
  const char* kn = static_cast<const char*>(a.k_new) + nbase * row_bytes;
  const char* vn = static_cast<const char*>(a.v_new) + nbase * row_bytes;
  // Two pieces per thread, held in named registers across the arrival.
  const int64_t i1 = i0 + stride;
  const uint4 k0 = *reinterpret_cast<const uint4*>(kn + min(i0, total - 1) * 16);
  const uint4 v0 = *reinterpret_cast<const uint4*>(vn + min(i0, total - 1) * 16);
  const uint4 k1 = *reinterpret_cast<const uint4*>(kn + min(i1, total - 1) * 16);
  const uint4 v1 = *reinterpret_cast<const uint4*>(vn + min(i1, total - 1) * 16);
  const Arrival av = arrive(a.unshared_len, a.active, a.slot_base, r, nblk, a.T_max);
  const int t = av.t;
  if (!av.grow) return;
  // Beam b's row goes to slot sb + b: piece i (beam i / pieces) keeps its
  // offset within the [B] block of rows.
  const int64_t sb = av.sbase + (int64_t)t * B;
  char* kp = static_cast<char*>(a.k_pool) + sb * row_bytes;
  char* vp = static_cast<char*>(a.v_pool) + sb * row_bytes;
  if (i0 < total) {
    *reinterpret_cast<uint4*>(kp + i0 * 16) = k0;
    *reinterpret_cast<uint4*>(vp + i0 * 16) = v0;
  }
  if (i1 < total) {
    *reinterpret_cast<uint4*>(kp + i1 * 16) = k1;
    *reinterpret_cast<uint4*>(vp + i1 * 16) = v1;
  }
  // Pieces beyond kPieces per thread (only when kv_blocks hit its cap).
  for (int64_t i = i0 + kPieces * stride; i < total; i += stride) {
    *reinterpret_cast<uint4*>(kp + i * 16) = *reinterpret_cast<const uint4*>(kn + i * 16);
    *reinterpret_cast<uint4*>(vp + i * 16) = *reinterpret_cast<const uint4*>(vn + i * 16);
  }
}

}  // namespace

bool append_supported(const AppendArgs& a) {
  if (a.T_max >= (1 << kArrivalShift)) return false;
  const AppendPlan p = plan_append(a);
  return p.col_blocks + p.kv_blocks <= kMaxAppendBlocks;
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  if (a.R == 0) return hipSuccess;
  const AppendPlan p = plan_append(a);
  const size_t lds = (size_t)a.B * p.col_chunk * sizeof(int32_t);
  dim3 grid(a.R, p.col_blocks + p.kv_blocks);
  hipLaunchKernelGGL(append_kernel, grid, dim3(kAppendThreads), lds, st, a, p);
  return hipGetLastError();
}

}  // namespace xattn
