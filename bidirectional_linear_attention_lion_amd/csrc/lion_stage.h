// lion_stage.h -- staging of key/value rows into LDS for the LION attention kernels (gfx950).
//
// Rows [row0, row0 + nrows) of a row-major [L][D] bf16 or fp32 array are copied straight from global
// memory into LDS with global_load_lds_dwordx4 (16 bytes per lane, no VGPRs in between), so a
// workgroup can have a whole stage of keys and values in flight at once.  One such load writes the
// 64 lanes' 16-byte chunks to 64 consecutive 16-byte LDS slots; slot s of the tile holds chunk
// (s % CPK) ^ swz(row) of row s / CPK, an XOR swizzle that spreads the 16-byte reads of 16 different
// rows (matrix-core A/B fragments) and the transposed reads over distinct banks.  Rows at or past L
// are loaded from row L - 1 (always in bounds); kernels zero or ignore them.
//
// V^T fragments are read from the row-major value tile with ds_read_b64_tr_b16: lane a of a 16-lane
// group addresses row 4g + a/4 (g = that group), columns 16 ct + 4 (a % 4) .. + 3, and receives the
// four values of column 16 ct + a at rows 4g .. 4g + 3 -- the layout the A operand of O^T = V^T P^T
// needs for keys 4g + e.
#pragma once

#include "lion_device.h"

namespace lion {

typedef short v4i16 __attribute__((ext_vector_type(4)));

template <int D, typename T>
struct RowTile {
    static constexpr int VEC = 16 / (int)sizeof(T);   // elements per 16-byte chunk
    static constexpr int CPK = D / VEC;                // chunks per row
    // eight 16-byte chunks per row (bf16 d = 64): row & 7, under which both the 16-row fragment reads
    // (lane group g reading chunk 4 s + g) and the transposed reads below hit distinct banks (checked
    // with the SQ_LDS_BANK_CONFLICT counter); other widths: (row >> 1) & (CPK - 1)
    __device__ static __forceinline__ int swz(int row) { return CPK == 8 ? (row & 7) : (row >> 1) & (CPK - 1); }
    // element offset of (row, col) in the swizzled tile
    __device__ static __forceinline__ int off(int row, int col) {
        return row * D + (((col / VEC) ^ swz(row)) * VEC) + (col % VEC);
    }
};

// Issue the direct loads of `nrows` rows (nrows * CPK a multiple of 64) starting at global row `row0`
// into `tile`; waves share the 1 KiB load instructions round-robin.  Completion is observed with
// s_waitcnt vmcnt(0) followed by a workgroup barrier.
template <int D, typename T>
__device__ __forceinline__ void stage_rows(T *tile, const T *src, int row0, int nrows, int L, int wave, int nw,
                                           int lane) {
    using RT = RowTile<D, T>;
    const int ninst = nrows * RT::CPK / 64;
    for (int i = wave; i < ninst; i += nw) {
        const int slot = i * 64 + lane;
        const int row = slot / RT::CPK;
        const int c = (slot % RT::CPK) ^ RT::swz(row);
        const int grow = min(row0 + row, L - 1);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src + (size_t)grow * D + c * RT::VEC),
                                         (__attribute__((address_space(3))) void *)(tile + i * 64 * RT::VEC),
                                         16, 0, 0);
    }
}

// bf16 rows [row0, row0 + nrows) of a row-major [L][D] array into an fp32 tile (RowTile<D, float>
// layout), converted exactly on the way: each thread loads 16 bytes (eight bf16 values) and writes them
// as two 16-byte fp32 chunks.  Unlike stage_rows this passes through VGPRs, so the caller's barrier
// after it also completes the copy.  Rows at or past L are loaded from row L - 1, as above.
template <int D>
__device__ __forceinline__ void stage_rows_cvt(float *tile, const __bf16 *src, int row0, int nrows, int L, int tid,
                                               int nt) {
    using RT = RowTile<D, float>;
    constexpr int C8 = D / 8;   // 16-byte bf16 chunks per row
    for (int i = tid; i < nrows * C8; i += nt) {
        const int row = i / C8, c8 = i % C8;
        const int grow = min(row0 + row, L - 1);
        const u32x4 raw = ld16(src + (size_t)grow * D + 8 * c8);
        // whole-vector operations (element-wise bit_casts of vector elements have miscompiled)
        const u32x4 ev = raw << 16, od = raw & 0xFFFF0000u;   // even and odd elements as fp32 bits
        const u32x4 lo = __builtin_shufflevector(ev, od, 0, 4, 1, 5);
        const u32x4 hi = __builtin_shufflevector(ev, od, 2, 6, 3, 7);
        *reinterpret_cast<u32x4 *>(tile + RT::off(row, 8 * c8)) = lo;
        *reinterpret_cast<u32x4 *>(tile + RT::off(row, 8 * c8 + 4)) = hi;
    }
}

// Issue the direct loads of `kib` KiB starting at `src` (16-byte aligned) into LDS at `dst`; waves
// share the 1 KiB load instructions round-robin.
__device__ __forceinline__ void stage_flat(void *dst, const void *src, int kib, int wave, int nw, int lane) {
    for (int i = wave; i < kib; i += nw)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const char *>(src) + (size_t)i * 1024 + lane * 16,
                                         (__attribute__((address_space(3))) void *)(reinterpret_cast<char *>(dst) + i * 1024),
                                         16, 0, 0);
}

// One lane's 16 bytes at `src` into the LDS slot of its lane index: this wave's load writes lane i's
// bytes to dst + 16 i (lanes that do not execute it leave their slots alone).
__device__ __forceinline__ void load_lds16(void *dst, const void *src) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
}

// Wait for this wave's outstanding vector-memory loads (which includes its direct LDS loads):
// s_waitcnt vmcnt(0) in the gfx9 encoding (vmcnt bits 3:0 and 15:14 = 0, expcnt 6:4 and lgkmcnt
// 11:8 at their maxima, i.e. not waited on).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Four bf16 values of one value channel at four consecutive keys (see the header comment).
__device__ __forceinline__ bf16x4 read_tr_b16(const __bf16 *p) {
    v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

}  // namespace lion
