// fa2_device.h -- gfx950 device helpers shared by the forward and backward kernels.
//
// Matrix-core conventions (v_mfma_f32_32x32x16_bf16, wave64), verified on the
// hardware for the output layout:
//   A operand (32 x 16, row i, reduction index k): lane l holds row i = l % 32
//     and the 8 reduction elements of lane group g = l / 32.
//   B operand (16 x 32, reduction index k, column j): lane l holds column
//     j = l % 32 and the same 8 reduction elements of group g.
//   C/D (32 x 32 fp32, 16 registers): register r of lane l is element
//     (i = 8*(r/4) + 4*g + r%4, j = l % 32).
// The reduction elements a lane holds only have to agree between A and B,
// so every kernel here picks the reduction order that suits its operands.
//
// Element format.  Q, K, V, O, dO and the gradients are bf16 by default; the
// kernel sources compiled with FA2_F16=1 take and produce f16 instead (the same
// kernels: operands are 16-bit patterns moved through registers and LDS, and
// only the matrix-product instruction, the fp32 -> 16-bit packing and the
// 16-bit -> fp32 reads below depend on the format).  The two builds live in
// namespaces fa2 and fa2_f16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef FA2_F16
#define FA2_F16 0
#endif
#if FA2_F16
#define FA2_NS fa2_f16
#define FA2_MFMA_32X32X16 "v_mfma_f32_32x32x16_f16"
#else
#define FA2_NS fa2
#define FA2_MFMA_32X32X16 "v_mfma_f32_32x32x16_bf16"
#endif

namespace FA2_NS {

typedef __bf16 el8 __attribute__((ext_vector_type(8)));      // 8 elements: MFMA operand storage
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA2_LDS __attribute__((address_space(3)))
#define FA2_GLOBAL __attribute__((address_space(1)))

// Bit reinterpretation through by-value parameters.  Never apply
// __builtin_bit_cast directly to an element of an ext_vector_type value
// (`v[i]`): this compiler then reads element 0 whatever i is.
__device__ __forceinline__ float u32_as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t f32_as_u32(float x) { return __builtin_bit_cast(uint32_t, x); }

__device__ __forceinline__ f32x16 mfma32(el8 a, el8 b, f32x16 c) {
#if FA2_F16
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  c, 0, 0, 0);
#else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
#endif
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Two fp32 -> two packed elements, rounded to nearest even (bf16:
// v_cvt_pk_bf16_f32; f16: v_cvt_f16_f32 per value).
__device__ __forceinline__ uint32_t pack_el(float lo, float hi) {
#if FA2_F16
    f16x2 v = {(_Float16)lo, (_Float16)hi};
#else
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
#endif
    return __builtin_bit_cast(uint32_t, v);
}

// The element in bits 0..15 / 16..31 of a packed pair, as fp32 (exact).
__device__ __forceinline__ float lo_el_f32(uint32_t x) {
#if FA2_F16
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
#else
    return __builtin_bit_cast(float, x << 16);
#endif
}
__device__ __forceinline__ float hi_el_f32(uint32_t x) {
#if FA2_F16
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
#else
    return __builtin_bit_cast(float, x & 0xffff0000u);
#endif
}

__device__ __forceinline__ el8 as_el8(u32x4 v) { return __builtin_bit_cast(el8, v); }

// lo + hi of a packed bf16 pair added into an fp32 accumulator (v_dot2c_f32_bf16 with ones).
__device__ __forceinline__ float add_bf16_pair(uint32_t pair, float acc) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), ones, acc, false);
}

// Combine lane l with lane l ^ 32 (v_permlane32_swap of a register with itself
// yields {low half, low half} and {high half, high half}).
__device__ __forceinline__ float max_halves(float x) {
    const uint32_t u = f32_as_u32(x);
    auto pr = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t lo = pr[0], hi = pr[1];
    return fmaxf(u32_as_f32(lo), u32_as_f32(hi));
}
__device__ __forceinline__ float sum_halves(float x) {
    const uint32_t u = f32_as_u32(x);
    auto pr = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t lo = pr[0], hi = pr[1];
    return u32_as_f32(lo) + u32_as_f32(hi);
}

// Workgroup `idx` of one level of a query-tile grid (B * Hq workgroups per
// level) -> batch and query head.  Workgroups are dealt round-robin to the 8
// XCDs, so idx % 8 picks the XCD.  With G > 1 query heads per K/V head and
// B * Hkv a multiple of 8, the G heads of a K/V head get one residue (and so
// share one XCD's L2, with every level of those heads); otherwise consecutive
// ids walk the heads.  Either way the map is a bijection onto [0, B * Hq).
__device__ __forceinline__ void level_head(int idx, int Hq, int G, int B, int& b, int& hq) {
    const int Hkv = Hq / G;
    if (G > 1 && (B * Hkv) % 8 == 0) {
        const int x = idx & 7, r = idx >> 3;        // XCD and rank on it
        const int m = r % G, gi = (r / G) * 8 + x;  // head m of K/V head group gi
        b = gi / Hkv;
        hq = (gi - b * Hkv) * G + m;
    } else {
        b = idx / Hq;
        hq = idx - b * Hq;
    }
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Block-sparse tile list, built by one wave: for the blocks c < n_blk whose
// flags(c) (a lane's block; 0 = not needed, else a bit set of up to 3 bits)
// are non-zero, in increasing c, the entries of its two 64-wide tiles 2c and
// 2c + 1 as (tile | flags << 12); a block past an odd tile count holds only
// tile 2c.  Returns the number of entries (wave-uniform).  Tile indices must
// be below 4096.
template <typename Flags>
__device__ __forceinline__ int build_tile_list(FA2_LDS uint16_t* list, int n_blk, int n_tiles, int lane,
                                               Flags flags) {
    int count = 0;
    bool single = false;
    for (int c0 = 0; c0 < n_blk; c0 += 64) {
        const int c = c0 + lane;
        const int f = c < n_blk ? flags(c) : 0;
        const uint64_t m = __builtin_amdgcn_ballot_w64(f != 0);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (f != 0) {
            const int pos = count + 2 * (int)below;
            list[pos] = (uint16_t)((2 * c) | (f << 12));
            if (2 * c + 1 < n_tiles) list[pos + 1] = (uint16_t)((2 * c + 1) | (f << 12));
        }
        single = single || __builtin_amdgcn_ballot_w64(f != 0 && 2 * c + 1 >= n_tiles) != 0;
        count += 2 * __builtin_popcountll(m);
    }
    return single ? count - 1 : count;   // the single-tile block is the last entry
}

// Block-sparse tile list without flags, built by one wave: for the blocks
// c < n_blk whose pred(c) holds, in increasing c, the tiles TPB*c ..
// TPB*c + TPB - 1 that lie below n_tiles (only the last block can be short).
// Returns the number of entries (wave-uniform).  Tile indices fit 16 bits.
template <int TPB, typename Pred>
__device__ __forceinline__ int build_block_tiles(FA2_LDS uint16_t* list, int n_blk, int n_tiles, int lane,
                                                 Pred pred) {
    int count = 0, short_by = 0;
    for (int c0 = 0; c0 < n_blk; c0 += 64) {
        const int c = c0 + lane;
        const bool f = c < n_blk && pred(c);
        const uint64_t m = __builtin_amdgcn_ballot_w64(f);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (f) {
            const int pos = count + TPB * (int)below;
#pragma unroll
            for (int t = 0; t < TPB; ++t)
                if (TPB * c + t < n_tiles) list[pos + t] = (uint16_t)(TPB * c + t);
        }
        if (__builtin_amdgcn_ballot_w64(f && TPB * c + TPB > n_tiles) != 0) short_by = TPB * n_blk - n_tiles;
        count += TPB * __builtin_popcountll(m);
    }
    return count - short_by;
}

// 16-byte LDS load / store.
__device__ __forceinline__ u32x4 lds_load16(const FA2_LDS char* p) {
    return *reinterpret_cast<const FA2_LDS u32x4*>(p);
}
__device__ __forceinline__ void lds_store16(FA2_LDS char* p, u32x4 v) {
    *reinterpret_cast<FA2_LDS u32x4*>(p) = v;
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element (i % 4) of the 4 consecutive bf16 that lane
// 4*e + i/4 addressed, as its element e (e = 0..3).  Measured on gfx950.
__device__ __forceinline__ s16x4 lds_load_tr(const FA2_LDS char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<FA2_LDS s16x4*>(const_cast<FA2_LDS char*>(p)));
}

__device__ __forceinline__ el8 cat_tr(s16x4 a, s16x4 b) {
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(el8, v);
}

// Asynchronous copies from global memory into LDS (global_load_lds_*): lane i
// of the wave writes its bytes at lds + SIZE*i, read from gbase + voff (gbase
// and lds wave-uniform, voff per lane).  They are issued as inline assembly:
// the compiler's own wait insertion then treats in-flight copies as unknown,
// instead of draining every outstanding LDS read (lgkmcnt(0)) before each use
// as it does for the builtin.  The copies count in vmcnt only (measured on
// gfx950: an in-flight copy does not hold lgkmcnt), so readers wait with
// wait_vm_keep / wait_vm_all followed by a barrier.  Nothing else in these
// kernels uses M0.
__device__ __forceinline__ void copy_to_lds16(const void* gbase, uint32_t voff, const FA2_LDS void* lds) {
    const uint32_t m0 = (uint32_t)(uintptr_t)lds;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 ::"s"(m0), "v"(voff), "s"(gbase) : "memory");
}
__device__ __forceinline__ void copy_to_lds4(const void* gbase, uint32_t voff, const FA2_LDS void* lds) {
    const uint32_t m0 = (uint32_t)(uintptr_t)lds;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 ::"s"(m0), "v"(voff), "s"(gbase) : "memory");
}

// s_waitcnt vmcnt(0) / vmcnt(N): all / all but the N most recent vector-memory
// operations (including the copies above) done.
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
template <int N> __device__ __forceinline__ void wait_vm_keep() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS reuse that leaves global->LDS copies in flight:
// lgkmcnt(0), then s_barrier.  (A fenced barrier would also wait for every
// outstanding copy, since the compiler counts them as pending LDS writes.)
// Each wave waits for the copies that the next reads depend on with
// wait_vm_keep / wait_vm_all before calling this.  The memory clobber keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ u32x4 global_load16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace FA2_NS
