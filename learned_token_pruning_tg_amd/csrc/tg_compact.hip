// Row compaction (gather of kept rows) for gfx950.
//
// Method (lucasainews.com TokenGate article, section "작동 방식"): only the
// kept tokens continue above the gate, and nothing is built for the dropped
// ones.  This kernel moves the kept rows into a dense [n_kept, row] buffer:
// dst[i] = src[idx[i]].
//
// Design: a pure HBM stream.  Wide rows (>= 1 KiB, e.g. a 4 KiB bf16
// residual row) get one 256-thread work-group pass per row with 16-byte
// accesses, so each row is one fully coalesced read and write; narrow rows
// (e.g. 4-byte scores) are flattened so that consecutive lanes touch
// consecutive elements.  The grid is sized to a few waves of work-groups per
// compute unit and strides over the rows.
#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kThreads = 256;

// One work-group per row (grid-stride over rows); T is the access unit.
template <typename T>
__global__ __launch_bounds__(kThreads) void compact_wide_kernel(
    const int32_t* __restrict__ idx, int64_t n_kept, const char* __restrict__ src,
    int64_t src_rows, int64_t src_stride, int64_t units, char* __restrict__ dst,
    int64_t dst_stride) {
  for (int64_t r = blockIdx.x; r < n_kept; r += gridDim.x) {
    const int64_t s = idx[r];
    if (s < 0 || s >= src_rows) continue;
    const T* sp = reinterpret_cast<const T*>(src + s * src_stride);
    T* dp = reinterpret_cast<T*>(dst + r * dst_stride);
    for (int64_t u = threadIdx.x; u < units; u += kThreads) dp[u] = sp[u];
  }
}

// Flattened (row, unit) space for narrow rows; T is the access unit.
template <typename T>
__global__ __launch_bounds__(kThreads) void compact_narrow_kernel(
    const int32_t* __restrict__ idx, int64_t n_kept, const char* __restrict__ src,
    int64_t src_rows, int64_t src_stride, int64_t units, char* __restrict__ dst,
    int64_t dst_stride) {
  const int64_t total = n_kept * units;
  for (int64_t f = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; f < total;
       f += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t r = f / units, u = f - r * units;
    const int64_t s = idx[r];
    if (s < 0 || s >= src_rows) continue;
    reinterpret_cast<T*>(dst + r * dst_stride)[u] =
        reinterpret_cast<const T*>(src + s * src_stride)[u];
  }
}

template <typename T>
hipError_t launch_t(const int32_t* idx, int64_t n_kept, const void* src, int64_t src_rows,
                    int64_t src_stride, int64_t row_bytes, void* dst, int64_t dst_stride,
                    hipStream_t stream) {
  const int64_t units = row_bytes / static_cast<int64_t>(sizeof(T));
  const char* s = static_cast<const char*>(src);
  char* d = static_cast<char*>(dst);
  constexpr int64_t kMaxBlocks = 256 * 16;
  if (row_bytes >= 1024) {
    const int64_t blocks = n_kept < kMaxBlocks ? n_kept : kMaxBlocks;
    hipLaunchKernelGGL(compact_wide_kernel<T>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, idx, n_kept, s, src_rows, src_stride, units, d,
                       dst_stride);
  } else {
    const int64_t total = n_kept * units;
    int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    hipLaunchKernelGGL(compact_narrow_kernel<T>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, idx, n_kept, s, src_rows, src_stride, units, d,
                       dst_stride);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compact(const int32_t* kept_idx, int64_t n_kept, const void* src,
                          int64_t src_rows, int64_t src_stride, int64_t row_bytes, void* dst,
                          int64_t dst_stride, hipStream_t stream) {
  if (n_kept == 0 || row_bytes == 0) return hipSuccess;
  const uintptr_t align = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) |
                          static_cast<uintptr_t>(src_stride) |
                          static_cast<uintptr_t>(dst_stride) | static_cast<uintptr_t>(row_bytes);
  if ((align & 15u) == 0)
    return launch_t<u32x4>(kept_idx, n_kept, src, src_rows, src_stride, row_bytes, dst,
                           dst_stride, stream);
  if ((align & 3u) == 0)
    return launch_t<uint32_t>(kept_idx, n_kept, src, src_rows, src_stride, row_bytes, dst,
                              dst_stride, stream);
  return launch_t<uint8_t>(kept_idx, n_kept, src, src_rows, src_stride, row_bytes, dst,
                           dst_stride, stream);
}

}  // namespace tg
