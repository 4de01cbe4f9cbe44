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
// returns t (the low bits), and the last arrival stores t + 1. Nothing else
// reads unshared_len during the launch.
#include "device.h"
#include "kernels.h"

namespace xattn {

namespace {

constexpr int kAppendThreads = 256;
constexpr int kTableLdsInts = 8192;  // 32 KiB of staged table cells per workgroup
constexpr int kPieces = 2;           // 16-byte K (and V) pieces per thread

struct AppendPlan {
  int col_chunk;   // table columns per workgroup
  int col_blocks;  // workgroups per request for the table
  int kv_blocks;   // workgroups per request for the K/V copy
};

AppendPlan plan_append(const AppendArgs& a) {
  AppendPlan p;
  p.col_chunk = kTableLdsInts / a.B;
  if (p.col_chunk < 1) p.col_chunk = 1;
  if (p.col_chunk > a.T_max) p.col_chunk = a.T_max;
  p.col_blocks = (a.T_max + p.col_chunk - 1) / p.col_chunk;
  const int64_t pieces = (int64_t)a.B * a.Hkv * a.D * a.elem_bytes / 16;
  const int64_t kv = (pieces + kAppendThreads * kPieces - 1) / (kAppendThreads * kPieces);
  p.kv_blocks = (int)(kv < 1 ? 1 : (kv > kMaxAppendBlocks / 2 ? kMaxAppendBlocks / 2 : kv));
  return p;
}

// Arrive at request r's counter; returns t (this call's position) to every
// thread of the workgroup. The last of the request's nblk workgroups stores
// the new length.
__device__ __forceinline__ int arrive(int32_t* ulen, int r, int nblk, int T_max) {
  __shared__ int s_t;
  if (threadIdx.x == 0) {
    const int old = atomicAdd(ulen + r, 1 << kArrivalShift);
    const int t = old & ((1 << kArrivalShift) - 1);
    if ((old >> kArrivalShift) == nblk - 1) ulen[r] = t < T_max ? t + 1 : t;
    s_t = t;
  }
  __syncthreads();
  return s_t;
}

__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a, AppendPlan p) {
  extern __shared__ int32_t staged[];  // [B][col_chunk]
  const int r = blockIdx.x;
  const int y = blockIdx.y;
  if (a.active && !a.active[r]) return;  // uniform: no workgroup of r arrives
  const int nblk = p.col_blocks + p.kv_blocks;
  const int B = a.B;
  const int64_t nbase = (int64_t)r * B;

  if (y < p.col_blocks) {
    const int t = arrive(a.unshared_len, r, nblk, a.T_max);
    if (t >= a.T_max) return;  // full row: nothing is written
    const int c0 = y * p.col_chunk;
    const int c1 = min(t, c0 + p.col_chunk);
    const int nc = c1 - c0;
    if (nc > 0) {
      for (int i = threadIdx.x; i < B * nc; i += blockDim.x) {
        const int b = i / nc, c = i - b * nc;
        staged[b * p.col_chunk + c] = a.table_in[(nbase + b) * a.T_max + c0 + c];
      }
      __syncthreads();
      for (int i = threadIdx.x; i < B * nc; i += blockDim.x) {
        const int b = i / nc, c = i - b * nc;
        const int par = a.parent[nbase + b];
        a.table_out[(nbase + b) * a.T_max + c0 + c] = staged[par * p.col_chunk + c];
      }
    }
    if (y == 0) {
      const int64_t sb = a.slot_base[r] + (int64_t)t * B;
      for (int b = threadIdx.x; b < B; b += blockDim.x)
        a.table_out[(nbase + b) * a.T_max + t] = (int32_t)(sb + b);
    }
    return;
  }

  // K/V copy: 16-byte pieces of the request's [B][H_kv][D] rows. The source
  // pieces do not depend on t, so they are loaded while the arrival is in
  // flight.
  const int64_t row_bytes = (int64_t)a.Hkv * a.D * a.elem_bytes;
  const int64_t pieces = row_bytes / 16;
  const int64_t total = pieces * B;
  const int64_t stride = (int64_t)p.kv_blocks * blockDim.x;
  const int64_t i0 = (int64_t)(y - p.col_blocks) * blockDim.x + threadIdx.x;
  const char* kn = static_cast<const char*>(a.k_new) + nbase * row_bytes;
  const char* vn = static_cast<const char*>(a.v_new) + nbase * row_bytes;
  uint4 kv[kPieces], vv[kPieces];
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    const int64_t i = i0 + j * stride;
    if (i < total) {
      kv[j] = *reinterpret_cast<const uint4*>(kn + i * 16);
      vv[j] = *reinterpret_cast<const uint4*>(vn + i * 16);
    }
  }
  const int t = arrive(a.unshared_len, r, nblk, a.T_max);
  if (t >= a.T_max) return;
  // Beam b's row goes to slot sb + b: piece i (beam i / pieces) keeps its
  // offset within the [B] block of rows.
  const int64_t sb = a.slot_base[r] + (int64_t)t * B;
  char* kp = static_cast<char*>(a.k_pool) + sb * row_bytes;
  char* vp = static_cast<char*>(a.v_pool) + sb * row_bytes;
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    const int64_t i = i0 + j * stride;
    if (i < total) {
      *reinterpret_cast<uint4*>(kp + i * 16) = kv[j];
      *reinterpret_cast<uint4*>(vp + i * 16) = vv[j];
    }
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
