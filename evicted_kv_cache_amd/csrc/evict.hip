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

// Copy `bytes` (a multiple of 2) from src to dst in the widest aligned unit.
__device__ __forceinline__ void copy_row(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int bytes) {
    if ((bytes & 15) == 0) {
        for (int o = 0; o < bytes; o += 16)
            *reinterpret_cast<uint4*>(dst + o) = *reinterpret_cast<const uint4*>(src + o);
    } else if ((bytes & 7) == 0) {
        for (int o = 0; o < bytes; o += 8)
            *reinterpret_cast<uint2*>(dst + o) = *reinterpret_cast<const uint2*>(src + o);
    } else if ((bytes & 3) == 0) {
        for (int o = 0; o < bytes; o += 4)
            *reinterpret_cast<uint32_t*>(dst + o) = *reinterpret_cast<const uint32_t*>(src + o);
    } else {
        for (int o = 0; o < bytes; o += 2)
            *reinterpret_cast<uint16_t*>(dst + o) = *reinterpret_cast<const uint16_t*>(src + o);
    }
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

// Thread (row, u) copies 16-byte unit u of every slot-indexed buffer whose row
// has that many units (code rows are multiples of 16 bytes); unit 0 also
// copies the shorter rows (per-token metadata) and the slot's position (per
// (b, h) position rows; for shared positions (0, 0, i) moves pos[i]), and
// (0, 0, i) moves k_row[i].  Consecutive threads touch consecutive units.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void gather_kernel(EvictArgs a, int upr) {
    const int m = a.sink + a.window;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t r = idx / upr;
    const int u = (int)(idx - r * upr);
    if (r >= (int64_t)a.BH * m) return;
    const int64_t bh = r / m;
    const int i = (int)(r - bh * m);
    const int si = i < a.sink ? i : a.n - a.window + (i - a.sink);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (k >= a.n_buf) break;
        const int rb = a.row_bytes[k];
        const uint8_t* src = static_cast<const uint8_t*>(a.src[k]) + (bh * a.cap + si) * rb;
        uint8_t* dst = static_cast<uint8_t*>(a.dst[k]) + (bh * a.cap + i) * rb;
        if ((rb & 15) == 0) {
            // each row is read and written once: non-temporal on both sides
            if (u * 16 < rb)
                __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(src + u * 16)),
                                            reinterpret_cast<u32x4v*>(dst + u * 16));
        } else if (u == 0) {
            copy_row(src, dst, rb);
        }
    }
    if (u == 0 && a.pos_per_head) a.dst_pos[bh * a.cap + i] = a.src_pos[bh * a.cap + si];
    if (bh == 0 && u == 0) {
        if (!a.pos_per_head) a.dst_pos[i] = a.src_pos[si];
        if (a.src_row && i < a.n_quant_new) {
            const RowRemap rr = row_remap(a.src_row, a.n, a.sink, a.window);
            const int old = a.src_row[si];
            a.dst_row[i] = i < a.sink ? old : old - rr.w_first + rr.base;
        }
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

}  // namespace

hipError_t launch_evict(const EvictArgs& a, hipStream_t s) {
    hipError_t e;
    int upr = 1;                                   // 16-byte units of the widest row
    for (int k = 0; k < a.n_buf; ++k) upr = a.row_bytes[k] / 16 > upr ? a.row_bytes[k] / 16 : upr;
    const int64_t threads = (int64_t)a.BH * (a.sink + a.window) * upr;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a, upr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.src_row) {
        const int n_quant_old = a.n_quant_new + (a.n - (a.sink + a.window));
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
