// evict.hip -- StreamingLLM sink + window compaction (gfx950).
//
// "StreamingLLM + KIVI", section "Implementation": once more than
// sink + window slots are stored, keep slots [0, sink) and the last `window`
// slots in order.  Here the compaction is an out-of-place gather: new slot i
// reads old slot i (i < sink) or n - window + (i - sink).  Every slot-indexed
// buffer (codes, per-token metadata, positions) is copied row by row in the
// widest aligned unit; nothing is re-quantized.
//
// KIVI per-channel keys: the scale table rows of token groups that no kept
// slot refers to are dropped (the page: per-channel K scales are not sliced by
// eviction, only rows are dropped).  The kept coded slots form two runs whose
// old rows are contiguous ranges [0, a_rows) and [w_first, w_last]; the new
// table is run A's rows followed by run W's rows (sharing one row when both
// runs touch the same group).  The four row ids are read on the device from
// the source k_row, so the host needs no read-back.
#include "kvq_internal.h"

namespace kvq {
namespace {

template <typename U>
__global__ __launch_bounds__(256) void gather_rows_kernel(const U* __restrict__ src, U* __restrict__ dst,
                                                          int units_per_row, int BH, int cap, int n,
                                                          int sink, int window) {
    const int m = sink + window;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)BH * m * units_per_row;
    if (idx >= total) return;
    const int64_t r = idx / units_per_row;
    const int u = (int)(idx - r * units_per_row);
    const int64_t bh = r / m;
    const int i = (int)(r - bh * m);
    const int si = i < sink ? i : n - window + (i - sink);
    dst[(bh * cap + i) * units_per_row + u] = src[(bh * cap + si) * units_per_row + u];
}

struct RowRemap {
    int a_rows;    // rows of the sink run (0 .. a_rows-1 unchanged)
    int w_first;   // first old row of the window run
    int base;      // new row id of w_first
};

__device__ __forceinline__ RowRemap row_remap(const int32_t* k_row, int n, int sink, int window) {
    RowRemap r;
    r.w_first = k_row[n - window];
    if (sink > 0) {
        const int a_last = k_row[sink - 1];
        r.a_rows = a_last + 1;
        r.base = (r.w_first == a_last) ? a_last : a_last + 1;
    } else {
        r.a_rows = 0;
        r.base = 0;
    }
    return r;
}

__global__ __launch_bounds__(256) void pos_rows_kernel(EvictArgs a) {
    const int m = a.sink + a.window;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= m) return;
    const int si = i < a.sink ? i : a.n - a.window + (i - a.sink);
    a.dst_pos[i] = a.src_pos[si];
    if (a.src_row && i < a.n_quant_new) {
        const RowRemap r = row_remap(a.src_row, a.n, a.sink, a.window);
        const int old = a.src_row[si];
        a.dst_row[i] = i < a.sink ? old : old - r.w_first + r.base;
    }
}

// Table rows: new row nr copies old row nr (nr < a_rows) or
// w_first + (nr - base) for nr < base + (w_last - w_first + 1).
__global__ __launch_bounds__(256) void table_kernel(EvictArgs a, int n_quant_old) {
    const RowRemap r = row_remap(a.src_row, a.n, a.sink, a.window);
    const int w_last = a.src_row[n_quant_old - 1];
    const int new_rows = r.base + (w_last - r.w_first + 1);
    const int upr = a.table_row_bytes / 16;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)a.BH * a.rows * upr;
    if (idx >= total) return;
    const int64_t rr = idx / upr;
    const int u = (int)(idx - rr * upr);
    const int64_t bh = rr / a.rows;
    const int nr = (int)(rr - bh * a.rows);
    if (nr >= new_rows) return;
    const int src_r = nr < r.a_rows ? nr : r.w_first + (nr - r.base);
    const uint4* s = static_cast<const uint4*>(a.src_table);
    uint4* d = static_cast<uint4*>(a.dst_table);
    d[(bh * a.rows + nr) * upr + u] = s[(bh * a.rows + src_r) * upr + u];
}

__global__ __launch_bounds__(256) void copy16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                     size_t n16) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) dst[i] = src[i];
}

template <typename U>
hipError_t gather(const void* src, void* dst, int row_bytes, const EvictArgs& a, hipStream_t s) {
    const int upr = row_bytes / (int)sizeof(U);
    const int64_t total = (int64_t)a.BH * (a.sink + a.window) * upr;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL((gather_rows_kernel<U>), dim3(blocks), dim3(256), 0, s,
                       static_cast<const U*>(src), static_cast<U*>(dst), upr, a.BH, a.cap, a.n,
                       a.sink, a.window);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_evict(const EvictArgs& a, hipStream_t s) {
    hipError_t e;
    for (int k = 0; k < a.n_buf; ++k) {
        const int rb = a.row_bytes[k];
        if (rb % 16 == 0) e = gather<uint4>(a.src[k], a.dst[k], rb, a, s);
        else if (rb % 8 == 0) e = gather<uint2>(a.src[k], a.dst[k], rb, a, s);
        else if (rb % 4 == 0) e = gather<uint32_t>(a.src[k], a.dst[k], rb, a, s);
        else if (rb % 2 == 0) e = gather<uint16_t>(a.src[k], a.dst[k], rb, a, s);
        else e = gather<uint8_t>(a.src[k], a.dst[k], rb, a, s);
        if (e != hipSuccess) return e;
    }
    const int m = a.sink + a.window;
    hipLaunchKernelGGL(pos_rows_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.src_row) {
        const int n_quant_old = a.n_quant_new + (a.n - m);
        const int64_t total = (int64_t)a.BH * a.rows * (a.table_row_bytes / 16);
        hipLaunchKernelGGL(table_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a,
                           n_quant_old);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const size_t n16 = a.resid_bytes / 16;
        hipLaunchKernelGGL(copy16_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                           static_cast<const uint4*>(a.src_resid), static_cast<uint4*>(a.dst_resid), n16);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kvq
