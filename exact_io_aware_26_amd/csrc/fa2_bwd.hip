// fa2_bwd.hip -- FlashAttention-2 backward pass for gfx950.
//
// Method (FlashAttention-2 summary page, zhaifeiyue.github.io, section 2
// "Q2 method" and section 3): the outer loop runs over K/V column blocks,
// one workgroup each; the inner loop streams the query row blocks (and, for
// GQA/MQA, the query heads sharing the K/V head, whose dK/dV are summed --
// section 4 checks); contributions to dQ from different K/V blocks meet in
// global memory through atomic adds (section 7).  P is not stored by the
// forward pass: it is rebuilt as P = exp(S - L) from the logsumexp L
// (section 4, "logsumexp fusion"), and D = rowsum(dO o O) (section 4 symbol
// table) replaces the row sums of dP o P.  The remaining formulas follow
// from differentiating O = softmax(scale * Q K^T) V:
//     dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
//     dK = scale * dS^T Q,  dQ = scale * dS K.
//
// Kernels, launched on one stream by fa2_bwd:
//   bwd_pre          -D = -rowsum(dO o O) and L log2(e) per padded row (fp32);
//                    in the atomic mode it also zeroes the fp32 dQ accumulator.
//   bwd_kv           d = 64, 128: one workgroup per 128 keys; dK and dV stay in
//                    registers over all query tiles (and all query heads of a
//                    GQA group).
//   bwd_dq_pipe      d = 64, 128: one workgroup per 256 query rows (128 with a
//                    block mask: one mask row); dQ stays in registers over all
//                    key blocks, recomputing S and dP, so no atomics are needed
//                    and dQ is deterministic.
//   bwd_kv256f       d = 256: the K/V loop with 32-row query tiles (dK, dV of
//                    the whole head dim in AGPRs).
//   bwd_dq256        d = 256: the dQ pass with 32-key tiles.
//   bwd_main         d = 256 in the atomic mode: the K/V loop with
//                    register-staged tiles and atomically added dQ.
//   bwd_pair         the pages' atomic accumulation of dQ for d = 64, 128
//   bwd_dq_convert   (FA2_BWD_DQ_ATOMIC), then dQ = bf16(scale * accumulator).
//
// gfx950 mapping shared by the K/V loops (each wave owns 32 keys of the tile,
// the backward analogue of splitting Q across waves):
//   * S = Q K_w^T and dP = dO V_w^T on v_mfma_f32_32x32x16_bf16 with the
//     wave's K_w / V_w rows as the B operand: every accumulator register then
//     holds one key per lane and 16 query rows, so P, dS and both gradient
//     accumulators share one register layout and need no data movement.
//   * dV^T += dO^T P and dK^T += Q^T dS take P and dS straight from registers
//     (as bf16) and read dO^T / Q^T fragments with ds_read_b64_tr_b16 from
//     row-major LDS tiles.
//   * In the atomic mode dQ needs dS with the queries across lanes, so each
//     wave writes its dS^T block to LDS; after one barrier the waves split the
//     dQ tile and add their fp32 results into the accumulator with global
//     atomics (one per element per K/V tile).
//   * LDS tiles use one XOR swizzle of the 16-byte chunks that is free of
//     bank conflicts both for 16-byte row reads (MFMA operands) and for the
//     transposed reads.
#include <type_traits>

#include <algorithm>

#include "fa2_device.h"
#include "fa2_kernels.h"

namespace FA2_NS {

namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kInf = __builtin_huge_valf();

// Swizzle of the 16-byte chunk index of an LDS row holding RB bytes.  The
// LDS serves a 16-byte-per-lane read 16 lanes per clock and an 8-byte read
// 32 lanes per clock (64 banks x 4 bytes).  Rows are read either as 16
// consecutive rows x one chunk (MFMA row operands) or as 4 consecutive rows
// x 4 chunks (transposed reads); this XOR pattern puts both on 64 distinct
// banks for 64-, 128-, 256- and 512-byte rows.
template <int RB> __device__ __forceinline__ int swz(int row) {
    return RB == 64 ? ((row >> 2) & 3)
         : RB == 128 ? 4 * ((row >> 1) & 1) + ((row >> 2) & 3)
                     : 4 * (row & 3) + ((row >> 2) & 3);
}

// Byte offset of element `col` (bf16) in row `row` of a swizzled tile with RB bytes per row.
template <int RB> __device__ __forceinline__ int tile_off(int row, int col) {
    return row * RB + 16 * ((col >> 3) ^ swz<RB>(row)) + 2 * (col & 7);
}

// A 32x16 (or 16x32) MFMA operand whose reduction index runs along the rows
// of a row-major LDS tile: two transposed reads (rows r0.. and r0+8..).
template <int RB>
__device__ __forceinline__ el8 tr_operand(const FA2_LDS char* tile, int r0, int c0, int lane) {
    const int j16 = lane & 15;
    const int g = lane >> 5;
    const int row = r0 + 4 * g + (j16 >> 2);
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);
    const s16x4 a = lds_load_tr(tile + tile_off<RB>(row, col));
    const s16x4 b = lds_load_tr(tile + tile_off<RB>(row + 8, col));
    return cat_tr(a, b);
}

// A row operand: lane holds row r0 + lane%32, 8 consecutive columns c0 + 8*(lane/32).
template <int RB>
__device__ __forceinline__ el8 row_operand(const FA2_LDS char* tile, int r0, int c0, int lane) {
    const int row = r0 + (lane & 31);
    const int col = c0 + 8 * (lane >> 5);
    return as_el8(lds_load16(tile + tile_off<RB>(row, col)));
}

// bwd_main (d = 256 only): BC keys per workgroup (32 per wave), BR query rows
// per inner tile; K_w/V_w MFMA operands live in VGPRs (KV_REGS) or are re-read
// from LDS.
template <int D> struct BwdCfg;
template <> struct BwdCfg<256> { static constexpr int BC = 64, NW = 2, BR = 32; static constexpr bool KV_REGS = false; };

// ---------------------------------------------------------------------------------------------
// bwd_pre: per padded row of each head, D_i = sum_d dO_id * O_id (fp32; with
// Olo, O_id + Olo_id, the forward's fp32 output to about 16 bits) and
// L_i * log2(e); rows past N get D = 0 and +inf (so P = 0 there), and so do
// rows whose L is -inf (block-sparse rows without an unmasked key).  Zeroes the
// dQ accumulator row when dQ is accumulated with atomics.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const BwdParams p, long rows_pad, int zero_dq) {
    constexpr int LPR = D / 8;                 // lanes per row (8 bf16 each)
    constexpr int RPB = 256 / LPR;             // rows per block
    const long rp = (long)blockIdx.x * RPB + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    const long bh = rp / p.Npad;
    const int qi = (int)(rp - bh * p.Npad);
    const bool valid = rp < rows_pad && qi < p.N;
    const long row = bh * p.N + qi;            // unpadded row (valid rows only)
    float acc = 0.f;
    if (valid) {
        const size_t off = (size_t)row * D + part * 8;
        const u32x4 a = global_load16(p.dO + off);
        const u32x4 b = global_load16(p.O + off);
        const u32x4 r = p.Olo ? global_load16(p.Olo + off) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t x = a[i], y = b[i], z = r[i];
            acc = fmaf(lo_el_f32(x), lo_el_f32(y) + lo_el_f32(z), acc);
            acc = fmaf(hi_el_f32(x), hi_el_f32(y) + hi_el_f32(z), acc);
        }
        if (zero_dq) {
            float* z = p.dQacc + off;
            *reinterpret_cast<u32x4*>(z) = u32x4{0, 0, 0, 0};
            *reinterpret_cast<u32x4*>(z + 4) = u32x4{0, 0, 0, 0};
        }
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
    if (rp < rows_pad && part == 0) {
        p.Dneg[rp] = -acc;
        const float l = valid ? p.L[row] : -kInf;
        p.L2[rp] = l != -kInf ? l * kLog2e : kInf;
    }
}

// ---------------------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool DQ_ATOMIC>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * BwdCfg<D>::NW, 64 * BwdCfg<D>::NW),
                          amdgpu_waves_per_eu(1, 1)))
void bwd_main_kernel(const BwdParams p) {
    constexpr int BC = BwdCfg<D>::BC;
    constexpr int NW = BwdCfg<D>::NW;
    constexpr bool KV_REGS = BwdCfg<D>::KV_REGS;
    constexpr int NT = 64 * NW;
    constexpr int BR = BwdCfg<D>::BR;
    constexpr int RB_D = 2 * D;        // bytes per row of Q/dO/K/V tiles
    constexpr int RB_Q = 2 * BR;       // bytes per row of the dS^T tile
    constexpr int KSD = D / 16;        // reduction steps over the head dim
    constexpr int NBD = D / 32;        // 32-wide head-dim blocks
    constexpr int NQB = BR / 32;       // 32-row query blocks per tile
    constexpr int KSKV = BC / 16;      // reduction steps over the keys of the workgroup
    constexpr int kKBytes = BC * RB_D;
    constexpr int kVBytes = KV_REGS ? 0 : BC * RB_D;
    constexpr int kQBytes = BR * RB_D;
    constexpr int kSBytes = BC * RB_Q;
    __shared__ __attribute__((aligned(16))) char smem_raw[kKBytes + kVBytes + 2 * kQBytes + 2 * kSBytes + 2 * BR * 4];
    FA2_LDS char* Ks = (FA2_LDS char*)smem_raw;
    FA2_LDS char* Vs = Ks + kKBytes;
    FA2_LDS char* Qs = Vs + kVBytes;
    FA2_LDS char* dOs = Qs + kQBytes;
    FA2_LDS char* dStBuf = dOs + kQBytes;      // two dS^T tiles: dQ runs one query tile behind
    FA2_LDS float* Ls = (FA2_LDS float*)(dStBuf + 2 * kSBytes);
    FA2_LDS float* Dl = Ls + BR;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 5;
    const int li = lane & 31;

    // ---- work item: the causal K/V tiles with the most query tiles first
    const int BHk = p.B * p.Hkv;
    const int kvtile = blockIdx.x / BHk;
    const int bh = blockIdx.x - kvtile * BHk;
    const int b = bh / p.Hkv;
    const int hk = bh - b * p.Hkv;
    const int N = p.N;
    const int kv0 = kvtile * BC;
    const int kw0 = kv0 + 32 * wave;          // this wave's first key
    const int kv = kw0 + li;                  // this lane's key
    const size_t khead = ((size_t)b * p.Hkv + hk) * (size_t)N * D;

    // ---- K (and V) tile of the workgroup into LDS; K_w / V_w into VGPRs
    {
        constexpr int CPR = D / 8;
        for (int c = tid; c < BC * CPR; c += NT) {
            const int row = c / CPR, col = (c % CPR) * 8;
            u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
            if (kv0 + row < N) {
                kx = global_load16(p.K + khead + (size_t)(kv0 + row) * D + col);
                if (!KV_REGS) vx = global_load16(p.V + khead + (size_t)(kv0 + row) * D + col);
            }
            lds_store16(Ks + tile_off<RB_D>(row, col), kx);
            if (!KV_REGS) lds_store16(Vs + tile_off<RB_D>(row, col), vx);
        }
    }
    el8 kf[KV_REGS ? KSD : 1], vf[KV_REGS ? KSD : 1];
    if (KV_REGS) {
#pragma unroll
        for (int ks = 0; ks < (KV_REGS ? KSD : 1); ++ks) {
            u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
            if (kv < N) {
                kx = global_load16(p.K + khead + (size_t)kv * D + 16 * ks + 8 * g);
                vx = global_load16(p.V + khead + (size_t)kv * D + 16 * ks + 8 * g);
            }
            kf[ks] = as_el8(kx);
            vf[ks] = as_el8(vx);
        }
    }

    f32x16 dv[NBD], dk[NBD];
#pragma unroll
    for (int i = 0; i < NBD; ++i) {
        dv[i] = zero16();
        dk[i] = zero16();
    }

    // ---- inner loop over (query head of the group, query tile)
    const int n_qt = (N + BR - 1) / BR;
    const int i_begin = CAUSAL ? kv0 / BR : 0;
    const int n_i = n_qt - i_begin;
    const int n_iter = n_i * p.G;

    // Next query tile staged in VGPRs (global -> VGPR -> LDS) while the current
    // one is computed, when that takes few registers per thread; otherwise the
    // tile is loaded straight into LDS at the top of its iteration.
    constexpr int QCH = BR * D / 8;                     // 16-byte chunks per Q tile
    constexpr int QPT = (QCH + NT - 1) / NT;
    constexpr bool PREFETCH = QPT <= 4;
    u32x4 sq[PREFETCH ? QPT : 1], so[PREFETCH ? QPT : 1];
    float sl = 0.f, sd = 0.f;

    auto stage = [&](int it) {
        const int hq = hk * p.G + it / n_i;
        const int qt0 = (i_begin + it % n_i) * BR;
        const size_t qhead = ((size_t)b * p.Hq + hq) * (size_t)N * D;
        if (PREFETCH) {
#pragma unroll
            for (int k = 0; k < (PREFETCH ? QPT : 1); ++k) {
                const int c = tid + k * NT;
                sq[k] = u32x4{0, 0, 0, 0};
                so[k] = u32x4{0, 0, 0, 0};
                if (c < QCH) {
                    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
                    if (qt0 + row < N) {
                        sq[k] = global_load16(p.Q + qhead + (size_t)(qt0 + row) * D + col);
                        so[k] = global_load16(p.dO + qhead + (size_t)(qt0 + row) * D + col);
                    }
                }
            }
        } else {
            for (int c = tid; c < QCH; c += NT) {
                const int row = c / (D / 8), col = (c % (D / 8)) * 8;
                u32x4 xq = {0, 0, 0, 0}, xo = {0, 0, 0, 0};
                if (qt0 + row < N) {
                    xq = global_load16(p.Q + qhead + (size_t)(qt0 + row) * D + col);
                    xo = global_load16(p.dO + qhead + (size_t)(qt0 + row) * D + col);
                }
                lds_store16(Qs + tile_off<RB_D>(row, col), xq);
                lds_store16(dOs + tile_off<RB_D>(row, col), xo);
            }
        }
        if (tid < BR) {
            // Raw values from a clamped row; scaled and masked when written to LDS,
            // so nothing here waits for these loads to land.
            const size_t r = ((size_t)b * p.Hq + hq) * (size_t)p.Npad + min(qt0 + tid, N - 1);
            sl = p.L2[r];
            sd = -p.Dneg[r];
        }
    };

    // dQ of query tile `it` (BR x D): the waves split the 32x32 output blocks and
    // reduce over all BC keys of the workgroup (dS^T and K by transposed LDS
    // reads), then add into the fp32 accumulator with one atomic per element.
    // Every wave issues the same fixed number of atomics: rows past the end
    // carry exactly +0 (their P is 0) and go to the last valid row.
    static_assert((NQB * NBD) % NW == 0, "dQ blocks must split evenly over the waves");
    auto dq_tile = [&](int it) {
        const int hq = hk * p.G + it / n_i;
        const int qt0 = (i_begin + it % n_i) * BR;
        const FA2_LDS char* dSt = dStBuf + (it & 1) * kSBytes;
        float* const dqh = p.dQacc + ((size_t)b * p.Hq + hq) * (size_t)N * D;   // uniform base
        const bool full = qt0 + BR <= N;
#pragma unroll
        for (int tt = 0; tt < NQB * NBD / NW; ++tt) {
            const int t = wave + tt * NW;
            const int qb = t / NBD, db = t % NBD;
            f32x16 acc = zero16();
            int kk_end = KSKV;
            if (CAUSAL) {
                // keys beyond the block's last query contribute dS = 0
                const int last_q = qt0 + 32 * qb + 31 - kv0;
                kk_end = min(KSKV, last_q / 16 + 1);
            }
            for (int kk = 0; kk < kk_end; ++kk) {
                const el8 a = tr_operand<RB_Q>(dSt, 16 * kk, 32 * qb, lane);
                const el8 bk = tr_operand<RB_D>(Ks, 16 * kk, 32 * db, lane);
                acc = mfma32(a, bk, acc);
            }
            const int d = 32 * db + li;
            const int row0 = qt0 + 32 * qb + 4 * g;
            if (full) {
                float* const base = dqh + (size_t)row0 * D + d;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    atomicAdd(base + (8 * (r >> 2) + (r & 3)) * D, acc[r]);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qg = min(row0 + 8 * (r >> 2) + (r & 3), N - 1);
                    atomicAdd(dqh + (size_t)qg * D + d, acc[r]);
                }
            }
        }
    };

    if (PREFETCH && n_iter > 0) stage(0);

    for (int it = 0; it < n_iter; ++it) {
        const int qt0 = (i_begin + it % n_i) * BR;

        // 1. query tile -> LDS (all waves are past barrier (B) of the previous
        //    iteration, so nobody still reads Q/dO/L/D of the previous tile)
        if (PREFETCH) {
#pragma unroll
            for (int k = 0; k < (PREFETCH ? QPT : 1); ++k) {
                const int c = tid + k * NT;
                if (c < QCH) {
                    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
                    lds_store16(Qs + tile_off<RB_D>(row, col), sq[k]);
                    lds_store16(dOs + tile_off<RB_D>(row, col), so[k]);
                }
            }
        } else {
            stage(it);
        }
        if (tid < BR) {
            const bool in = qt0 + tid < N;
            Ls[tid] = in ? sl : kInf;                  // rows past the end get P = 0
            Dl[tid] = in ? sd : 0.f;
        }
        __syncthreads();                               // (A) tile visible

        // 2. dQ of the previous tile (its dS^T is complete since barrier (B)); its
        //    atomics, then the next tile's loads, get all of step 3 to land.
        if (DQ_ATOMIC && it > 0) dq_tile(it - 1);
        if (PREFETCH && it + 1 < n_iter) stage(it + 1);
        FA2_LDS char* dSt = dStBuf + (it & 1) * kSBytes;

        // 3. Per 32-row query block: S, dP (MFMA), P, dS (VALU), dS^T -> LDS, then
        //    dV^T += dO^T P and dK^T += Q^T dS.  Every wave always runs (keys a
        //    query tile cannot see get P = 0 from the mask), so the gradient
        //    accumulators are updated unconditionally.
        const bool need_mask = (CAUSAL && qt0 < kw0 + 32) || qt0 + BR > N || kw0 + 32 > N;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const el8 aq = row_operand<RB_D>(Qs, 32 * qb, 16 * ks, lane);
                const el8 ao = row_operand<RB_D>(dOs, 32 * qb, 16 * ks, lane);
                el8 bk, bv;
                if (KV_REGS) {
                    bk = kf[KV_REGS ? ks : 0];
                    bv = vf[KV_REGS ? ks : 0];
                } else {
                    bk = row_operand<RB_D>(Ks, 32 * wave, 16 * ks, lane);
                    bv = row_operand<RB_D>(Vs, 32 * wave, 16 * ks, lane);
                }
                s = mfma32(aq, bk, s);
                dp = mfma32(ao, bv, dp);
            }
            if (need_mask) {
                // keys above the diagonal or past the end: S = -inf, so P = 0
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qg = qt0 + 32 * qb + 8 * (r >> 2) + 4 * g + (r & 3);
                    if ((CAUSAL && kv > qg) || kv >= N) s[r] = -kInf;
                }
            }
            uint32_t pp[8], sp[8];
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int ql = 32 * qb + 8 * rq + 4 * g;          // local query of register 4*rq
                const f32x4 lv = *reinterpret_cast<const FA2_LDS f32x4*>(Ls + ql);
                const f32x4 dd = *reinterpret_cast<const FA2_LDS f32x4*>(Dl + ql);
                float pr[4], dsr[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * rq + e;
                    pr[e] = exp2_fast(fmaf(s[r], p.c, -lv[e]));
                    dsr[e] = pr[e] * (dp[r] - dd[e]);
                }
                pp[2 * rq] = pack_el(pr[0], pr[1]);
                pp[2 * rq + 1] = pack_el(pr[2], pr[3]);
                sp[2 * rq] = pack_el(dsr[0], dsr[1]);
                sp[2 * rq + 1] = pack_el(dsr[2], dsr[3]);
                // dS^T[key][query .. query+3]
                *reinterpret_cast<FA2_LDS u32x2*>(dSt + tile_off<RB_Q>(32 * wave + li, ql)) =
                    u32x2{sp[2 * rq], sp[2 * rq + 1]};
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int kk = 2 * qb + h;
                const el8 bp = as_el8(u32x4{pp[4 * h], pp[4 * h + 1], pp[4 * h + 2], pp[4 * h + 3]});
                const el8 bs = as_el8(u32x4{sp[4 * h], sp[4 * h + 1], sp[4 * h + 2], sp[4 * h + 3]});
#pragma unroll
                for (int db = 0; db < NBD; ++db) {
                    const el8 ao = tr_operand<RB_D>(dOs, 16 * kk, 32 * db, lane);
                    dv[db] = mfma32(ao, bp, dv[db]);
                    const el8 aq = tr_operand<RB_D>(Qs, 16 * kk, 32 * db, lane);
                    dk[db] = mfma32(aq, bs, dk[db]);
                }
            }
        }
        __syncthreads();                               // (B) dS^T visible; Q/dO/L/D free

    }
    if (DQ_ATOMIC && n_iter > 0) dq_tile(n_iter - 1);

    // ---- epilogue: dV, dK (scaled) for this lane's key
    if (kv < N) {
        uint16_t* dVr = p.dV + khead + (size_t)kv * D;
        uint16_t* dKr = p.dK + khead + (size_t)kv * D;
#pragma unroll
        for (int db = 0; db < NBD; ++db)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int d0 = 32 * db + 8 * rq + 4 * g;
                *reinterpret_cast<u32x2*>(dVr + d0) =
                    u32x2{pack_el(dv[db][4 * rq], dv[db][4 * rq + 1]),
                          pack_el(dv[db][4 * rq + 2], dv[db][4 * rq + 3])};
                *reinterpret_cast<u32x2*>(dKr + d0) =
                    u32x2{pack_el(dk[db][4 * rq] * p.scale, dk[db][4 * rq + 1] * p.scale),
                          pack_el(dk[db][4 * rq + 2] * p.scale, dk[db][4 * rq + 3] * p.scale)};
            }
    }
}

// ---------------------------------------------------------------------------------------------
// bwd_pair: the K/V-tile loop for d = 64 and 128 with two waves per SIMD.
//
// Eight waves form four pairs; pair k owns keys 32k..32k+31 of the 128-key
// tile.  For each 64-row query tile, wave h of a pair (h = 0, 1) computes S,
// dP, P and dS for query block h (32 rows, full head dim) and publishes P and
// dS to LDS; then each wave accumulates dV and dK for ITS HALF of the head
// dim from both query blocks.  So no MFMA is duplicated, the gradient
// accumulators take half the registers, and two waves fit on every SIMD
// (one MFMA stream can run while the other wave does softmax or LDS work).
//
// P^T and dS^T tiles are stored [key][query] with the query columns of every
// 16-group in bit-swapped order (bits 2 and 3 exchanged): then a plain
// 16-byte row read returns exactly the 8 queries a lane must hold as the
// MFMA B operand, in the order of the transposed-read A operands
// (4g + 0..3, 8 + 4g + 0..3 within a 16-query step).  dQ reads dS^T with
// transposed reads, so its output rows come out in that swapped order and
// the atomics map them back.
//
// Two barriers per query tile: Q/dO/L/D are double-buffered, dS^T is
// double-buffered (dQ runs one tile behind), P^T is single-buffered (it is
// consumed before the next tile's first barrier).
__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

template <int D, bool CAUSAL, bool DQ_ATOMIC>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void bwd_pair_kernel(const BwdParams p) {
    constexpr int BC = 128, NT = 512, BR = 64;
    constexpr int RB_D = 2 * D;        // bytes per row of K / Q / dO tiles
    constexpr int RB_Q = 2 * BR;       // bytes per row of the P^T / dS^T tiles
    constexpr int KSD = D / 16;        // reduction steps over the head dim (S, dP)
    constexpr int NBH = D / 64;        // 32-wide head-dim blocks per half
    constexpr int KSKV = BC / 16;      // reduction steps over the keys (dQ)
    constexpr int NBD = D / 32;        // 32-wide head-dim blocks (dQ)
    constexpr int kKBytes = BC * RB_D;
    constexpr int kQBytes = BR * RB_D;
    constexpr int kSBytes = BC * RB_Q;
    __shared__ __attribute__((aligned(16))) char smem_raw[kKBytes + 4 * kQBytes + 3 * kSBytes + 4 * BR * 4];
    FA2_LDS char* Ks = (FA2_LDS char*)smem_raw;
    FA2_LDS char* QObuf = Ks + kKBytes;             // [2][Q tile, dO tile]
    FA2_LDS char* dStBuf = QObuf + 4 * kQBytes;     // [2] dS^T
    FA2_LDS char* Pt = dStBuf + 2 * kSBytes;        // P^T
    FA2_LDS float* LDbuf = (FA2_LDS float*)(Pt + kSBytes);  // [2][L row, D row]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 5;
    const int li = lane & 31;
    const int kvb = wave & 3;          // key block of the pair
    const int h = wave >> 2;           // query block (phase A) and head-dim half (phase B)

    const int BHk = p.B * p.Hkv;
    const int kvtile = blockIdx.x / BHk;
    const int bh = blockIdx.x - kvtile * BHk;
    const int b = bh / p.Hkv;
    const int hk = bh - b * p.Hkv;
    const int N = p.N;
    const int kv0 = kvtile * BC;
    const int kw0 = kv0 + 32 * kvb;
    const int kv = kw0 + li;
    const size_t khead = ((size_t)b * p.Hkv + hk) * (size_t)N * D;

    // K tile -> LDS (dQ operand); this pair's K/V rows -> VGPRs (S, dP operands)
    {
        constexpr int CPR = D / 8;
        for (int c = tid; c < BC * CPR; c += NT) {
            const int row = c / CPR, col = (c % CPR) * 8;
            u32x4 kx = {0, 0, 0, 0};
            if (kv0 + row < N) kx = global_load16(p.K + khead + (size_t)(kv0 + row) * D + col);
            lds_store16(Ks + tile_off<RB_D>(row, col), kx);
        }
    }
    el8 kf[KSD], vf[KSD];
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
        u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
        if (kv < N) {
            kx = global_load16(p.K + khead + (size_t)kv * D + 16 * ks + 8 * g);
            vx = global_load16(p.V + khead + (size_t)kv * D + 16 * ks + 8 * g);
        }
        kf[ks] = as_el8(kx);
        vf[ks] = as_el8(vx);
    }
    f32x16 dv[NBH], dk[NBH];
#pragma unroll
    for (int i = 0; i < NBH; ++i) {
        dv[i] = zero16();
        dk[i] = zero16();
    }

    const int n_qt = (N + BR - 1) / BR;
    const int i_begin = CAUSAL ? kv0 / BR : 0;
    const int n_i = n_qt - i_begin;
    const int n_iter = n_i * p.G;

    // Next query tile staged in VGPRs while the current one is computed.
    constexpr int QCH = BR * D / 8;
    constexpr int QPT = QCH / NT;
    static_assert(QPT >= 1 && QCH % NT == 0, "query tile / threads mismatch");
    u32x4 sq[QPT], so[QPT];
    float sl = 0.f, sd = 0.f;
    auto stage = [&](int it) {
        const int hq = hk * p.G + it / n_i;
        const int qt0 = (i_begin + it % n_i) * BR;
        const size_t qhead = ((size_t)b * p.Hq + hq) * (size_t)N * D;
#pragma unroll
        for (int k = 0; k < QPT; ++k) {
            const int c = tid + k * NT;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
            sq[k] = u32x4{0, 0, 0, 0};
            so[k] = u32x4{0, 0, 0, 0};
            if (qt0 + row < N) {
                sq[k] = global_load16(p.Q + qhead + (size_t)(qt0 + row) * D + col);
                so[k] = global_load16(p.dO + qhead + (size_t)(qt0 + row) * D + col);
            }
        }
        if (tid < BR) {   // raw values from a clamped row; scaled and masked when stored
            const size_t r = ((size_t)b * p.Hq + hq) * (size_t)p.Npad + min(qt0 + tid, N - 1);
            sl = p.L2[r];
            sd = p.Dneg[r];
        }
    };

    // dQ of query tile `it`: one 32x32 output block per wave (d = 128; waves 0-3
    // for d = 64), reduced over the 128 keys; one atomic per element.
    constexpr int NDQ = 2 * NBD;       // output blocks per query tile
    auto dq_tile = [&](int it) {
        if (wave >= NDQ) return;
        const int hq = hk * p.G + it / n_i;
        const int qt0 = (i_begin + it % n_i) * BR;
        const FA2_LDS char* dSt = dStBuf + (it & 1) * kSBytes;
        const int qb = wave & 1, db = wave >> 1;
        f32x16 acc = zero16();
        int kk_end = KSKV;
        if (CAUSAL) kk_end = min(KSKV, (qt0 + 32 * qb + 31 - kv0) / 16 + 1);
        for (int kk = 0; kk < kk_end; ++kk) {
            const el8 a = tr_operand<RB_Q>(dSt, 16 * kk, 32 * qb, lane);
            const el8 bk = tr_operand<RB_D>(Ks, 16 * kk, 32 * db, lane);
            acc = mfma32(a, bk, acc);
        }
        // Output row i = 8*(r/4) + 4g + r%4 holds dS^T column i, i.e. query swap23(i).
        float* const dqh = p.dQacc + ((size_t)b * p.Hq + hq) * (size_t)N * D;
        const int d = 32 * db + li;
        const int row0 = qt0 + 32 * qb + 8 * g;
        if (qt0 + BR <= N) {
            float* const base = dqh + (size_t)row0 * D + d;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                atomicAdd(base + (16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3)) * D, acc[r]);
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qg = min(row0 + 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3), N - 1);
                atomicAdd(dqh + (size_t)qg * D + d, acc[r]);   // rows past the end add +0
            }
        }
    };

    if (n_iter > 0) stage(0);
    for (int it = 0; it < n_iter; ++it) {
        const int qt0 = (i_begin + it % n_i) * BR;
        const int buf = it & 1;
        FA2_LDS char* Qs = QObuf + buf * 2 * kQBytes;
        FA2_LDS char* dOs = Qs + kQBytes;
        FA2_LDS float* Ls = LDbuf + buf * 2 * BR;
        FA2_LDS float* Dl = Ls + BR;
        FA2_LDS char* dSt = dStBuf + buf * kSBytes;

        // 1. staged tile -> LDS buffer `buf` (last read two tiles ago)
#pragma unroll
        for (int k = 0; k < QPT; ++k) {
            const int c = tid + k * NT;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
            lds_store16(Qs + tile_off<RB_D>(row, col), sq[k]);
            lds_store16(dOs + tile_off<RB_D>(row, col), so[k]);
        }
        if (tid < BR) {
            const bool in = qt0 + tid < N;
            Ls[tid] = in ? sl : kInf;   // rows past the end get P = 0
            Dl[tid] = in ? sd : 0.f;   // -D
        }
        __syncthreads();                         // (A)

        // 2. dQ of the previous tile, then the next tile's loads; both land during 3-4.
        if (DQ_ATOMIC && it > 0) dq_tile(it - 1);
        if (it + 1 < n_iter) stage(it + 1);

        // 3. query block h: S, dP, P, dS for this pair's keys; publish P^T, dS^T.
        {
            // dP starts from -D (four consecutive queries per load, in register
            // order), so the products end at dP - D.
            f32x16 s = zero16(), dp;
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const f32x4 nd = *reinterpret_cast<const FA2_LDS f32x4*>(Dl + 32 * h + 8 * rq + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) dp[4 * rq + e] = nd[e];
            }
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const el8 aq = row_operand<RB_D>(Qs, 32 * h, 16 * ks, lane);
                const el8 ao = row_operand<RB_D>(dOs, 32 * h, 16 * ks, lane);
                s = mfma32(aq, kf[ks], s);
                dp = mfma32(ao, vf[ks], dp);
            }
            const bool need_mask = (CAUSAL && qt0 + 32 * h < kw0 + 32) || qt0 + 32 * h + 32 > N || kw0 + 32 > N;
            if (need_mask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qg = qt0 + 32 * h + 8 * (r >> 2) + 4 * g + (r & 3);
                    if ((CAUSAL && kv > qg) || kv >= N) s[r] = -kInf;
                }
            }
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int ql = 32 * h + 8 * rq + 4 * g;          // local query of register 4*rq
                const f32x4 lv = *reinterpret_cast<const FA2_LDS f32x4*>(Ls + ql);
                float pr[4], dsr[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * rq + e;
                    pr[e] = exp2_fast(fmaf(s[r], p.c, -lv[e]));
                    dsr[e] = pr[e] * dp[r];
                }
                const int pos = 32 * h + swap23(8 * rq + 4 * g);   // 4 queries stay contiguous
                const int off = tile_off<RB_Q>(32 * kvb + li, pos);
                *reinterpret_cast<FA2_LDS u32x2*>(Pt + off) = u32x2{pack_el(pr[0], pr[1]), pack_el(pr[2], pr[3])};
                *reinterpret_cast<FA2_LDS u32x2*>(dSt + off) = u32x2{pack_el(dsr[0], dsr[1]), pack_el(dsr[2], dsr[3])};
            }
        }
        __syncthreads();                         // (X) P^T, dS^T of both query blocks visible

        // 4. dV^T += dO^T P and dK^T += Q^T dS over both query blocks, this wave's half of d.
#pragma unroll
        for (int kk = 0; kk < BR / 16; ++kk) {
            const int row = 32 * kvb + li;
            const int col = 16 * kk + 8 * g;
            const el8 bp = as_el8(lds_load16(Pt + tile_off<RB_Q>(row, col)));
            const el8 bs = as_el8(lds_load16(dSt + tile_off<RB_Q>(row, col)));
#pragma unroll
            for (int j = 0; j < NBH; ++j) {
                const int dcol = (D / 2) * h + 32 * j;
                const el8 ao = tr_operand<RB_D>(dOs, 16 * kk, dcol, lane);
                dv[j] = mfma32(ao, bp, dv[j]);
                const el8 aq = tr_operand<RB_D>(Qs, 16 * kk, dcol, lane);
                dk[j] = mfma32(aq, bs, dk[j]);
            }
        }
    }
    if (DQ_ATOMIC && n_iter > 0) {
        __syncthreads();                         // dS^T of the last tile complete
        dq_tile(n_iter - 1);
    }

    // epilogue: this lane's key, this wave's half of the head dim
    if (kv < N) {
        uint16_t* dVr = p.dV + khead + (size_t)kv * D;
        uint16_t* dKr = p.dK + khead + (size_t)kv * D;
#pragma unroll
        for (int j = 0; j < NBH; ++j)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int d0 = (D / 2) * h + 32 * j + 8 * rq + 4 * g;
                *reinterpret_cast<u32x2*>(dVr + d0) =
                    u32x2{pack_el(dv[j][4 * rq], dv[j][4 * rq + 1]),
                          pack_el(dv[j][4 * rq + 2], dv[j][4 * rq + 3])};
                *reinterpret_cast<u32x2*>(dKr + d0) =
                    u32x2{pack_el(dk[j][4 * rq] * p.scale, dk[j][4 * rq + 1] * p.scale),
                          pack_el(dk[j][4 * rq + 2] * p.scale, dk[j][4 * rq + 3] * p.scale)};
            }
    }
}

// ---------------------------------------------------------------------------------------------
// bwd_dq_pipe: the dQ pass for d = 64 and 128.
//
// One workgroup = 4 wave64s, one wave per SIMD; each wave owns two 32-row query
// blocks (u = 0, 1; 256 rows per workgroup) at d = 128.  With a block mask it
// owns one block, so that a 128-row workgroup is one mask row; at d = 64 also
// one block, so that the kernel fits 256 registers and two workgroups share a
// CU (two waves per SIMD from independent workgroups: 3-9 % faster there).  Q and dO of its rows are MFMA B
// operands in registers and its dQ^T accumulators stay in registers, all
// transposed so that each lane owns one query row of each block:
//     s  = K Q^T,  dp = V dO^T          (A: K / V rows from LDS)
//     P  = exp2(c s - L log2 e),  dS = P o (dp - D)   (masked on the diagonal)
//     dQ^T += K^T dS^T                  (A: K^T by transposed reads, B: dS^T registers)
// Every A operand read from LDS feeds the products of both query blocks, and
// each K / V tile copied into LDS serves 256 query rows.  The keys the causal
// mask lets through are walked in 32-key blocks; 64-key tiles of K and V are
// copied into LDS four deep.  Stage s is a fixed program of operand loads,
// each followed by its two products: the s, dp loads of block s alternate
// (two to one) with the dQ loads of block s-2, while the dS of block s-1 is
// formed element by element over the stage's slots, so the vector work of a
// block runs beside the products of its neighbours.  A tile is read in four
// consecutive stages; one barrier per tile.  The first two stages read a
// zeroed "tile -1" and add nothing, and two stages more than there are blocks
// drain the pipeline.  The stage loop is unrolled by eight so that every
// buffer offset is a compile-time immediate.  The dQ^T accumulators (128
// registers at d = 128) live in AGPRs.
template <int D, bool CAUSAL, bool SPARSE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 1)))
void bwd_dq_pipe_kernel(const BwdParams p) {
    // Block-sparse: one query block per wave, so a workgroup (128 rows) is
    // one mask row and computes no tile that its rows do not need.
    constexpr int NW = 4, U = SPARSE || D == 64 ? 1 : 2, BRQ = 32 * U * NW, BT = 64;
    constexpr int RB = 2 * D;
    constexpr int kTile = BT * RB;
    constexpr int KSD = D / 16, NBD = D / 32;
    constexpr int NSD = 2 * KSD;                      // s, dp operand loads per block
    constexpr int NQ = 2 * NBD;                       // dQ operand loads per block
    constexpr int SL = NSD + NQ;                      // operand loads (pairs of products) per stage
    constexpr int RPI = 1024 / RB, CPR = RB / 16;
    constexpr int PERW = kTile / 1024 / NW;
    constexpr int NCOPY = 2 * PERW;
    constexpr int kPrefetch = 4;
    constexpr int NE = 16 * U;                        // dS elements per lane per block
    static_assert(NSD == 2 * NQ && PERW >= 1 && NCOPY <= SL && SL % kPrefetch == 0, "stage program shape");
    __shared__ __attribute__((aligned(256))) char Ka[4 * kTile], Va[4 * kTile];
    FA2_LDS char* const Kbuf = (FA2_LDS char*)Ka;
    FA2_LDS char* const Vbuf = (FA2_LDS char*)Va;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int li = lane & 31;

    const int n_qtiles = (p.N + BRQ - 1) / BRQ;
    const int BH = p.B * p.Hq;
    const int level = blockIdx.x / BH;
    const int bh = blockIdx.x - level * BH;
    const int qtile = n_qtiles - 1 - level;
    int b, hq;
    level_head(bh, p.Hq, p.G, p.B, b, hq);
    const int hk = hq / p.G;
    const int N = p.N;
    const size_t qhead = ((size_t)b * p.Hq + hq) * (size_t)N * D;
    const size_t khead = ((size_t)b * p.Hkv + hk) * (size_t)N * D;
    const int q0 = qtile * BRQ;
    const int wq0 = q0 + 32 * U * wave;

    el8 qf[U][KSD], of[U][KSD];
    float l2[U], dq_d[U];
    int qu[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int q = wq0 + 32 * u + li;
        qu[u] = q;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            u32x4 a = {0, 0, 0, 0}, c = {0, 0, 0, 0};
            if (q < N) {
                a = global_load16(p.Q + qhead + (size_t)q * D + 16 * ks + 8 * g);
                c = global_load16(p.dO + qhead + (size_t)q * D + 16 * ks + 8 * g);
            }
            qf[u][ks] = as_el8(a);
            of[u][ks] = as_el8(c);
        }
        const size_t row = ((size_t)b * p.Hq + hq) * (size_t)p.Npad + min(q, N - 1);
        l2[u] = q < N ? p.L2[row] : kInf;
        dq_d[u] = q < N ? -p.Dneg[row] : 0.f;
    }

    // 32-key blocks and 64-key tiles of the walk.  Block-sparse: the list
    // entries, the tiles of every key block that the workgroup's 128-row
    // mask block needs (causal: at or below its diagonal).
    int n_kb, n_t;
    FA2_LDS uint16_t* tl = nullptr;
    if constexpr (SPARSE) {
        static_assert(BRQ == kSparseBlock && 2 * BT == kSparseBlock, "one mask block, two tiles per block");
        __shared__ uint16_t tl_arr[kSparseMaxN / BT];
        __shared__ int tl_count;
        tl = (FA2_LDS uint16_t*)tl_arr;
        if (wave == 0) {
            const int r0 = q0 / kSparseBlock, nb = p.nb;
            const int n = build_tile_list(tl, nb, (N + BT - 1) / BT, lane, [&](int c) {
                return p.bmask[(size_t)r0 * nb + c] != 0 && (!CAUSAL || c <= r0) ? 1 : 0;
            });
            if (lane == 0) tl_count = n;
        }
        __syncthreads();
        n_t = __builtin_amdgcn_readfirstlane(tl_count);
        n_kb = 2 * n_t;
    } else {
        n_kb = CAUSAL ? (min(q0 + BRQ, N) - 1) / 32 + 1 : (N + 31) / 32;
        n_t = (n_kb + 1) / 2;
    }
    auto tile_at = [&](int t) -> int {
        if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)(tl[t] & 0xfff));
        else return t;
    };

    auto copy_part = [&](int t, int buf, int j) {
        const int kv0 = tile_at(min(t, n_t - 1)) * BT;
        const int last = N - 1 - kv0;
        const int i = j % PERW;
        const int R = (wave * PERW + i) * RPI;
        const int lr = lane / CPR;
        const int lc = 16 * ((lane % CPR) ^ swz<RB>(lane / CPR));
        const uint32_t off = (uint32_t)(min(R + lr, last) * RB + (lc ^ (16 * swz<RB>(R))));
        const uint16_t* src = (j < PERW ? p.K : p.V) + khead + (size_t)kv0 * D;
        copy_to_lds16(src, off, (j < PERW ? Kbuf : Vbuf) + buf * kTile + (wave * PERW + i) * 1024);
    };

    const int j16 = lane & 15;
    const int xq = 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1);
    const int r1 = 4 * g + (j16 >> 2), r2 = r1 + 8;
    const int kb_lane = li * RB + 16 * (g ^ swz<RB>(li));
    const int vb1_lane = r1 * RB + 8 * (j16 & 1) + 16 * (xq ^ swz<RB>(r1));
    const int vb2_lane = r2 * RB + 8 * (j16 & 1) + 16 * (xq ^ swz<RB>(r2));
    const FA2_LDS char* kp[KSD];
    const FA2_LDS char* vp[KSD];
    const FA2_LDS char* tp1[NBD];
    const FA2_LDS char* tp2[NBD];
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
        kp[ks] = Kbuf + (kb_lane ^ (32 * ks));
        vp[ks] = Vbuf + (kb_lane ^ (32 * ks));
        asm volatile("" : "+v"(kp[ks]), "+v"(vp[ks]));
    }
#pragma unroll
    for (int db = 0; db < NBD; ++db) {
        tp1[db] = Kbuf + (vb1_lane ^ (64 * db));
        tp2[db] = Kbuf + (vb2_lane ^ (64 * db));
        asm volatile("" : "+v"(tp1[db]), "+v"(tp2[db]));
    }

    f32x16 acc[U][NBD];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < NBD; ++i) acc[u][i] = zero16();
    f32x16 sc[2][U], dpc[2][U];
    uint32_t dsp[2][U][8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            sc[i][u] = zero16();
            dpc[i][u] = zero16();
#pragma unroll
            for (int r = 0; r < 8; ++r) dsp[i][u][r] = 0u;
        }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[1][u][r] = -kInf;

    el8 abuf[kPrefetch];           // operands loaded ahead of their products
    auto stage = [&](auto s8_tag, int s) __attribute__((always_inline)) {
        constexpr int S8 = decltype(s8_tag)::value;
        constexpr int P_SD = S8 & 1;
        constexpr int P_EL = P_SD ^ 1;
        // Operand load k of stage T8 (mod 8): block T8 lives in tile buffer
        // (T8 >> 1) & 3, block T8 - 2 in the buffer before it; both at rows
        // 32 * (T8 & 1).  Every offset is a compile-time immediate.
        auto load_at = [&](auto t8_tag, int k) -> el8 {
            constexpr int T8 = decltype(t8_tag)::value;
            constexpr int off_sd = ((T8 >> 1) & 3) * kTile + 32 * (T8 & 1) * RB;
            constexpr int off_q = (((T8 >> 1) + 3) & 3) * kTile + 32 * (T8 & 1) * RB;
            if (k % 3 != 2) {
                const int j = 2 * (k / 3) + k % 3, ks = j >> 1;
                return as_el8(lds_load16(((j & 1) ? vp[ks] : kp[ks]) + off_sd));
            }
            const int qq = k / 3, h = qq / NBD, db = qq % NBD;
            const int off = off_q + 16 * h * RB;
            return cat_tr(lds_load_tr(tp1[db] + off), lds_load_tr(tp2[db] + off));
        };
        auto load_a = [&](int k) { return load_at(s8_tag, k); };
        auto product = [&](int k, int u, el8 a) {
            if (k % 3 != 2) {
                const int j = 2 * (k / 3) + k % 3, ks = j >> 1;
                if (j & 1) dpc[P_SD][u] = mfma32(a, of[u][ks], ks == 0 ? zero16() : dpc[P_SD][u]);
                else sc[P_SD][u] = mfma32(a, qf[u][ks], ks == 0 ? zero16() : sc[P_SD][u]);
                return;
            }
            const int qq = k / 3, h = qq / NBD, db = qq % NBD;
            const el8 bds = as_el8(u32x4{dsp[P_SD][u][4 * h], dsp[P_SD][u][4 * h + 1],
                                               dsp[P_SD][u][4 * h + 2], dsp[P_SD][u][4 * h + 3]});
            // Issued as assembly to keep the accumulator in AGPRs (the compiler
            // places every builtin product's result in VGPRs here, which would
            // not fit); acc[u][db] is next touched a dozen products later.
            f32x16 c = acc[u][db];
            asm volatile(FA2_MFMA_32X32X16 " %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(bds));
            acc[u][db] = c;
        };
        auto pin = [](float& x) { asm volatile("" : "+v"(x)); };
        auto pin_u = [](uint32_t& x) { asm volatile("" : "+v"(x)); };
        auto el_a = [&](int e) {
            const int u = e >> 4, r = e & 15;
            float x = fmaf(sc[P_EL][u][r], p.c, -l2[u]);
            pin(x);
            sc[P_EL][u][r] = x;
        };
        auto el_b = [&](int e) {
            const int u = e >> 4, r = e & 15;
            float x = exp2_fast(sc[P_EL][u][r]);
            pin(x);
            sc[P_EL][u][r] = x;
        };
        auto el_c = [&](int e) {
            const int u = e >> 4, r = e & 15;
            float x = sc[P_EL][u][r] * (dpc[P_EL][u][r] - dq_d[u]);
            pin(x);
            dpc[P_EL][u][r] = x;
            if (r & 1) {
                uint32_t w = pack_el(dpc[P_EL][u][r - 1], x);
                pin_u(w);
                dsp[P_EL][u][r >> 1] = w;
            }
        };
        {
            // Block s - 1 (stages past the last block compute scores nobody reads).
            int kb0;
            if constexpr (SPARSE) {
                const int bi = min(max(s - 1, 0), n_kb - 1);
                const int e = __builtin_amdgcn_readfirstlane((int)tl[bi >> 1]);
                kb0 = (e & 0xfff) * BT + 32 * (bi & 1);
            } else {
                kb0 = 32 * (s - 1);
            }
            if ((CAUSAL && kb0 + 31 > wq0) || kb0 + 32 > N) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    // Element i holds key kb0 + 4g + 8 (i / 4) + i % 4: masked when
                    // that constant offset exceeds lim (one compare, one select).
                    const int lim = (CAUSAL ? min(qu[u], N - 1) : N - 1) - kb0 - 4 * g;
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        sc[P_EL][u][i] = 8 * (i >> 2) + (i & 3) > lim ? -kInf : sc[P_EL][u][i];
                }
            }
        }
        const bool copy_stage = (S8 & 1) == 0;
        constexpr int BUF_W = ((S8 >> 1) + 2) & 3;
        const int tcopy = (s >> 1) + 2;
        // An even stage and the odd one after it read the same tile (no barrier
        // between them), so the even stage loads the odd stage's first operands
        // in its last slots; operand k always goes to abuf[k % kPrefetch].
        constexpr bool kLoadedBefore = (S8 & 1) == 1;
        if constexpr (!kLoadedBefore) {
#pragma unroll
            for (int k = 0; k < kPrefetch; ++k) abuf[k] = load_a(k);
        }
        // 2 * SL product slots: load k feeds slots 2k (u = 0) and 2k + 1 (u = 1).
#pragma unroll
        for (int k = 0; k < SL; ++k) {
            const el8 a = abuf[k % kPrefetch];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                __builtin_amdgcn_sched_barrier(0);
                const int slot = U * k + u;
                if (u == 0 && k + kPrefetch < SL) abuf[k % kPrefetch] = load_a(k + kPrefetch);
                else if (u == 0 && copy_stage)
                    abuf[k % kPrefetch] = load_at(std::integral_constant<int, S8 + 1>{}, k + kPrefetch - SL);
                product(k, u, a);
#pragma unroll
                for (int e = 0; e < NE; ++e) {
                    const int sa = e * (U * SL - 3) / (NE - 1);
                    if (slot == sa + 2) el_c(e);
                    if (slot == sa + 1) el_b(e);
                    if (slot == sa) el_a(e);
                }
                if (copy_stage && slot >= 1 && slot <= NCOPY) copy_part(tcopy, BUF_W, slot - 1);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (!copy_stage) {
            wait_vm_keep<NCOPY>();
            barrier_lds();
        }
    };

    // A block-sparse workgroup with no tile only writes dQ = 0.
    if (!SPARSE || n_t > 0) {
    for (int i = tid; i < kTile / 16; i += 64 * NW) {
        lds_store16(Kbuf + 3 * kTile + 16 * i, u32x4{0, 0, 0, 0});
        lds_store16(Vbuf + 3 * kTile + 16 * i, u32x4{0, 0, 0, 0});
    }
#pragma unroll
    for (int j = 0; j < NCOPY; ++j) copy_part(0, 0, j);
#pragma unroll
    for (int j = 0; j < NCOPY; ++j) copy_part(1, 1, j);
    wait_vm_all();
    __syncthreads();
    const int n_stage = n_kb + 2;
    for (int s = 0; s < n_stage; s += 8) {
        stage(std::integral_constant<int, 0>{}, s);
        if (s + 1 < n_stage) stage(std::integral_constant<int, 1>{}, s + 1);
        if (s + 2 < n_stage) stage(std::integral_constant<int, 2>{}, s + 2);
        if (s + 3 < n_stage) stage(std::integral_constant<int, 3>{}, s + 3);
        if (s + 4 < n_stage) stage(std::integral_constant<int, 4>{}, s + 4);
        if (s + 5 < n_stage) stage(std::integral_constant<int, 5>{}, s + 5);
        if (s + 6 < n_stage) stage(std::integral_constant<int, 6>{}, s + 6);
        if (s + 7 < n_stage) stage(std::integral_constant<int, 7>{}, s + 7);
    }
    wait_vm_all();
    }
    // The accumulators were last written by matrix products issued from inline
    // assembly, which the compiler does not track: wait them out before reading.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int q = qu[u];
        if (q < N) {
            uint16_t* dQr = p.dQ + qhead + (size_t)q * D;
#pragma unroll
            for (int db = 0; db < NBD; ++db)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int d0 = 32 * db + 8 * rq + 4 * g;
                    *reinterpret_cast<u32x2*>(dQr + d0) =
                        u32x2{pack_el(acc[u][db][4 * rq] * p.scale, acc[u][db][4 * rq + 1] * p.scale),
                              pack_el(acc[u][db][4 * rq + 2] * p.scale, acc[u][db][4 * rq + 3] * p.scale)};
                }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// bwd_dq256: the pipelined dQ pass at d = 256.  One 32-row query block per
// wave (128 rows per workgroup); 32-key tiles of K and V (16 KiB each) copied
// into LDS four deep, one tile per stage, one barrier per stage.  Stage s runs
// the same program as bwd_dq_pipe's: the s, dp products of block s alternate
// with the dQ products of block s - 2, while the dS of block s - 1 is formed
// beside them.  The dQ^T accumulators and the Q / dO operands fill the AGPRs.
// Block-sparse (SPARSE): a workgroup is one 128-row mask block and walks the
// 32-key tiles of the key blocks its mask row keeps (causal: at or below the
// diagonal) from an LDS list.
template <bool CAUSAL, bool SPARSE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_dq256_kernel(const BwdParams p) {
    constexpr int D = 256;
    constexpr int NW = 4, U = 1, BRQ = 32 * U * NW, BT = 32;   // one 32-key block per tile
    constexpr int RB = 2 * D;
    constexpr int kTile = BT * RB;
    constexpr int KSD = D / 16, NBD = D / 32;
    constexpr int NSD = 2 * KSD;                      // s, dp operand loads per block
    constexpr int NQ = 2 * NBD;                       // dQ operand loads per block
    constexpr int SL = NSD + NQ;                      // operand loads (pairs of products) per stage
    constexpr int RPI = 1024 / RB, CPR = RB / 16;
    constexpr int PERW = kTile / 1024 / NW;
    constexpr int NCOPY = 2 * PERW;
    constexpr int kPrefetch = 4;
    constexpr int NE = 16 * U;                        // dS elements per lane per block
    static_assert(NSD == 2 * NQ && PERW >= 1 && NCOPY <= SL, "stage program shape");
    __shared__ __attribute__((aligned(256))) char Ka[4 * kTile], Va[4 * kTile];
    FA2_LDS char* const Kbuf = (FA2_LDS char*)Ka;
    FA2_LDS char* const Vbuf = (FA2_LDS char*)Va;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int li = lane & 31;

    const int n_qtiles = (p.N + BRQ - 1) / BRQ;
    const int BH = p.B * p.Hq;
    const int level = blockIdx.x / BH;
    const int bh = blockIdx.x - level * BH;
    const int qtile = n_qtiles - 1 - level;
    int b, hq;
    level_head(bh, p.Hq, p.G, p.B, b, hq);
    const int hk = hq / p.G;
    const int N = p.N;
    const size_t qhead = ((size_t)b * p.Hq + hq) * (size_t)N * D;
    const size_t khead = ((size_t)b * p.Hkv + hk) * (size_t)N * D;
    const int q0 = qtile * BRQ;
    const int wq0 = q0 + 32 * U * wave;

    el8 qf[U][KSD], of[U][KSD];
    float l2[U], dq_d[U];
    int qu[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int q = wq0 + 32 * u + li;
        qu[u] = q;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            u32x4 a = {0, 0, 0, 0}, c = {0, 0, 0, 0};
            if (q < N) {
                a = global_load16(p.Q + qhead + (size_t)q * D + 16 * ks + 8 * g);
                c = global_load16(p.dO + qhead + (size_t)q * D + 16 * ks + 8 * g);
            }
            qf[u][ks] = as_el8(a);
            of[u][ks] = as_el8(c);
        }
        const size_t row = ((size_t)b * p.Hq + hq) * (size_t)p.Npad + min(q, N - 1);
        l2[u] = q < N ? p.L2[row] : kInf;
        dq_d[u] = q < N ? -p.Dneg[row] : 0.f;
    }

    // 32-key tiles of the walk (one block per tile).  Block-sparse: the list
    // entries, the tiles of every key block the workgroup's mask block needs.
    int n_kb;
    FA2_LDS uint16_t* tl = nullptr;
    if constexpr (SPARSE) {
        static_assert(BRQ == kSparseBlock && kSparseBlock % BT == 0, "one mask block per workgroup");
        __shared__ uint16_t tl_arr[kSparseMaxN / BT];
        __shared__ int tl_count;
        tl = (FA2_LDS uint16_t*)tl_arr;
        if (wave == 0) {
            const int r0 = q0 / kSparseBlock, nb = p.nb;
            const int n = build_block_tiles<kSparseBlock / BT>(tl, nb, (N + BT - 1) / BT, lane, [&](int c) {
                return p.bmask[(size_t)r0 * nb + c] != 0 && (!CAUSAL || c <= r0);
            });
            if (lane == 0) tl_count = n;
        }
        __syncthreads();
        n_kb = __builtin_amdgcn_readfirstlane(tl_count);
    } else {
        n_kb = CAUSAL ? (min(q0 + BRQ, N) - 1) / 32 + 1 : (N + 31) / 32;
    }
    const int n_t = n_kb;
    auto tile_at = [&](int t) -> int {
        if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)tl[t]);
        else return t;
    };

    auto copy_part = [&](int t, int buf, int j) {
        const int kv0 = tile_at(min(t, n_t - 1)) * BT;
        const int last = N - 1 - kv0;
        const int i = j % PERW;
        const int R = (wave * PERW + i) * RPI;
        const int lr = lane / CPR;
        const int lc = 16 * ((lane % CPR) ^ swz<RB>(lane / CPR));
        const uint32_t off = (uint32_t)(min(R + lr, last) * RB + (lc ^ (16 * swz<RB>(R))));
        const uint16_t* src = (j < PERW ? p.K : p.V) + khead + (size_t)kv0 * D;
        copy_to_lds16(src, off, (j < PERW ? Kbuf : Vbuf) + buf * kTile + (wave * PERW + i) * 1024);
    };

    const int j16 = lane & 15;
    const int xq = 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1);
    const int r1 = 4 * g + (j16 >> 2), r2 = r1 + 8;
    const int kb_lane = li * RB + 16 * (g ^ swz<RB>(li));
    const int vb1_lane = r1 * RB + 8 * (j16 & 1) + 16 * (xq ^ swz<RB>(r1));
    const int vb2_lane = r2 * RB + 8 * (j16 & 1) + 16 * (xq ^ swz<RB>(r2));
    const FA2_LDS char* kp[KSD];
    const FA2_LDS char* vp[KSD];
    const FA2_LDS char* tp1[NBD];
    const FA2_LDS char* tp2[NBD];
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
        kp[ks] = Kbuf + (kb_lane ^ (32 * ks));
        vp[ks] = Vbuf + (kb_lane ^ (32 * ks));
        asm volatile("" : "+v"(kp[ks]), "+v"(vp[ks]));
    }
#pragma unroll
    for (int db = 0; db < NBD; ++db) {
        tp1[db] = Kbuf + (vb1_lane ^ (64 * db));
        tp2[db] = Kbuf + (vb2_lane ^ (64 * db));
        asm volatile("" : "+v"(tp1[db]), "+v"(tp2[db]));
    }

    f32x16 acc[U][NBD];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < NBD; ++i) acc[u][i] = zero16();
    f32x16 sc[2][U], dpc[2][U];
    uint32_t dsp[2][U][8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            sc[i][u] = zero16();
            dpc[i][u] = zero16();
#pragma unroll
            for (int r = 0; r < 8; ++r) dsp[i][u][r] = 0u;
        }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[1][u][r] = -kInf;

    el8 abuf[kPrefetch];           // operands loaded ahead of their products
    auto stage = [&](auto s4_tag, int s) __attribute__((always_inline)) {
        constexpr int S4 = decltype(s4_tag)::value;
        constexpr int P_SD = S4 & 1;
        constexpr int P_EL = P_SD ^ 1;
        // Operand load k of stage S4 (mod 4): block S4 is tile buffer S4, block
        // S4 - 2 the buffer two before it.  Every offset is a compile-time
        // immediate.
        auto load_a = [&](int k) -> el8 {
            constexpr int off_sd = (S4 & 3) * kTile;
            constexpr int off_q = ((S4 + 2) & 3) * kTile;
            if (k % 3 != 2) {
                const int j = 2 * (k / 3) + k % 3, ks = j >> 1;
                return as_el8(lds_load16(((j & 1) ? vp[ks] : kp[ks]) + off_sd));
            }
            const int qq = k / 3, h = qq / NBD, db = qq % NBD;
            const int off = off_q + 16 * h * RB;
            return cat_tr(lds_load_tr(tp1[db] + off), lds_load_tr(tp2[db] + off));
        };
        auto product = [&](int k, int u, el8 a) {
            if (k % 3 != 2) {
                const int j = 2 * (k / 3) + k % 3, ks = j >> 1;
                if (j & 1) dpc[P_SD][u] = mfma32(a, of[u][ks], ks == 0 ? zero16() : dpc[P_SD][u]);
                else sc[P_SD][u] = mfma32(a, qf[u][ks], ks == 0 ? zero16() : sc[P_SD][u]);
                return;
            }
            const int qq = k / 3, h = qq / NBD, db = qq % NBD;
            const el8 bds = as_el8(u32x4{dsp[P_SD][u][4 * h], dsp[P_SD][u][4 * h + 1],
                                               dsp[P_SD][u][4 * h + 2], dsp[P_SD][u][4 * h + 3]});
            // Issued as assembly to keep the accumulator in AGPRs (the compiler
            // places every builtin product's result in VGPRs here, which would
            // not fit); acc[u][db] is next touched a dozen products later.
            f32x16 c = acc[u][db];
            asm volatile(FA2_MFMA_32X32X16 " %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(bds));
            acc[u][db] = c;
        };
        auto pin = [](float& x) { asm volatile("" : "+v"(x)); };
        auto pin_u = [](uint32_t& x) { asm volatile("" : "+v"(x)); };
        auto el_a = [&](int e) {
            const int u = e >> 4, r = e & 15;
            float x = fmaf(sc[P_EL][u][r], p.c, -l2[u]);
            pin(x);
            sc[P_EL][u][r] = x;
        };
        auto el_b = [&](int e) {
            const int u = e >> 4, r = e & 15;
            float x = exp2_fast(sc[P_EL][u][r]);
            pin(x);
            sc[P_EL][u][r] = x;
        };
        auto el_c = [&](int e) {
            const int u = e >> 4, r = e & 15;
            float x = sc[P_EL][u][r] * (dpc[P_EL][u][r] - dq_d[u]);
            pin(x);
            dpc[P_EL][u][r] = x;
            if (r & 1) {
                uint32_t w = pack_el(dpc[P_EL][u][r - 1], x);
                pin_u(w);
                dsp[P_EL][u][r >> 1] = w;
            }
        };
        {
            // Block s - 1 (stages past the last block compute scores nobody reads).
            const int kb0 = SPARSE ? tile_at(min(max(s - 1, 0), n_kb - 1)) * BT : 32 * (s - 1);
            if ((CAUSAL && kb0 + 31 > wq0) || kb0 + 32 > N) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    // Element i holds key kb0 + 4g + 8 (i / 4) + i % 4: masked when
                    // that constant offset exceeds lim (one compare, one select).
                    const int lim = (CAUSAL ? min(qu[u], N - 1) : N - 1) - kb0 - 4 * g;
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        sc[P_EL][u][i] = 8 * (i >> 2) + (i & 3) > lim ? -kInf : sc[P_EL][u][i];
                }
            }
        }
        // Each stage copies the next tile into the buffer that the barrier
        // ending the previous stage released (block s - 3's).
        constexpr int BUF_W = (S4 + 1) & 3;
        const int tcopy = s + 1;
#pragma unroll
        for (int k = 0; k < kPrefetch; ++k) abuf[k] = load_a(k);
        // 2 * SL product slots: load k feeds slots 2k (u = 0) and 2k + 1 (u = 1).
#pragma unroll
        for (int k = 0; k < SL; ++k) {
            const el8 a = abuf[k % kPrefetch];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                __builtin_amdgcn_sched_barrier(0);
                const int slot = U * k + u;
                if (u == 0 && k + kPrefetch < SL) abuf[k % kPrefetch] = load_a(k + kPrefetch);
                product(k, u, a);
#pragma unroll
                for (int e = 0; e < NE; ++e) {
                    const int sa = e * (U * SL - 3) / (NE - 1);
                    if (slot == sa + 2) el_c(e);
                    if (slot == sa + 1) el_b(e);
                    if (slot == sa) el_a(e);
                }
                if (slot >= 1 && slot <= NCOPY) copy_part(tcopy, BUF_W, slot - 1);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_all();                                    // tile s + 1 has landed
        barrier_lds();
    };

    // A block-sparse workgroup with no tile only writes dQ = 0.
    if (!SPARSE || n_kb > 0) {
    // Prologue: tile 0; the buffers of tiles -2 and -1 zeroed.
    for (int i = tid; i < 2 * kTile / 16; i += 64 * NW) {
        lds_store16(Kbuf + 2 * kTile + 16 * i, u32x4{0, 0, 0, 0});
        lds_store16(Vbuf + 2 * kTile + 16 * i, u32x4{0, 0, 0, 0});
    }
#pragma unroll
    for (int j = 0; j < NCOPY; ++j) copy_part(0, 0, j);
    wait_vm_all();
    __syncthreads();
    const int n_stage = n_kb + 2;
    for (int s = 0; s < n_stage; s += 4) {
        stage(std::integral_constant<int, 0>{}, s);
        if (s + 1 < n_stage) stage(std::integral_constant<int, 1>{}, s + 1);
        if (s + 2 < n_stage) stage(std::integral_constant<int, 2>{}, s + 2);
        if (s + 3 < n_stage) stage(std::integral_constant<int, 3>{}, s + 3);
    }
    wait_vm_all();
    }
    // The accumulators were last written by matrix products issued from inline
    // assembly, which the compiler does not track: wait them out before reading.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int q = qu[u];
        if (q < N) {
            uint16_t* dQr = p.dQ + qhead + (size_t)q * D;
#pragma unroll
            for (int db = 0; db < NBD; ++db)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int d0 = 32 * db + 8 * rq + 4 * g;
                    *reinterpret_cast<u32x2*>(dQr + d0) =
                        u32x2{pack_el(acc[u][db][4 * rq] * p.scale, acc[u][db][4 * rq + 1] * p.scale),
                              pack_el(acc[u][db][4 * rq + 2] * p.scale, acc[u][db][4 * rq + 3] * p.scale)};
                }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// bwd_kv: the K/V-tile loop for d = 64 and 128 (dQ in its own pass).
//
// One workgroup = 4 wave64s = 128 keys; wave w owns keys 32w..32w+31 and the
// whole head dim of their dK and dV, accumulated in registers (at d = 128 one
// wave per SIMD with the full register file; at d = 64 two workgroups per CU).  Query tiles of 64 rows -- Q, dO, and
// the L log2(e) and D rows of the workspace -- are copied into LDS with
// global_load_lds, three tiles deep, in nine distinct LDS arrays with the loop
// unrolled by three (no read names a buffer in flight; each step waits only
// for the copies issued one step earlier).  Per 32-row query block every
// product is arranged so that each lane owns one key:
//     s  = Q K^T,  dp = dO V^T     A: Q / dO rows from LDS, B: this lane's K / V row
//     P  = exp2(c s - L log2 e),   dS = P o (dp - D)      (masked on the diagonal)
//     dV^T += dO^T P,  dK^T += Q^T dS
//                                  A: dO^T / Q^T by transposed LDS reads,
//                                  B: P / dS straight from the s / dp registers,
// since a score accumulator register holds the 8 queries, in the order of the
// transposed reads, that the B operand of a 16-query step needs.  Within a
// tile, the vector work of one query block overlaps the products of the next.
// NB query blocks per tile: 2 (64-row tiles), or 4 for causal d = 128 when N
// is a multiple of 128 (128-row tiles, so a tile's fixed costs -- barrier,
// waits, copies, the operand pipeline's restart -- spread over twice the
// products; the workspace rows are padded to 64 only, so the 128-row tiles
// must not pass N).  Two such tiles fill the LDS, so the ring is two deep
// there.  At d = 64 the kernel fits 256 registers and runs two workgroups per
// CU (two waves per SIMD from independent workgroups), which beat 128-row
// tiles at one wave per SIMD by 3-6 %.
template <int D, bool CAUSAL, bool SPARSE, int NB>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(D == 64 && NB == 2 ? 2 : 1, D == 64 && NB == 2 ? 2 : 1)))
void bwd_kv_kernel(const BwdParams p) {
    static_assert(NB == 2 || (NB == 4 && !SPARSE), "tile shapes");
    constexpr int NW = 4, BC = 32 * NW, BR = 32 * NB;
    constexpr int RB = 2 * D;                 // bytes per row of the Q / dO tiles
    constexpr int kTile = BR * RB;
    constexpr int KSD = D / 16;               // reduction steps over the head dim
    constexpr int NBD = D / 32;               // 32-wide head-dim blocks
    constexpr int RPI = 1024 / RB;            // tile rows per wave copy instruction
    constexpr int CPR = RB / 16;              // 16-byte chunks per row
    constexpr int PERW = kTile / 1024 / NW;   // copy instructions per wave per tensor
    static_assert(BR % kBwdRowPad == 0 && PERW >= 1 && kTile % (1024 * NW) == 0, "tile / waves mismatch");
    // One LDS array per buffered query tile, [Q | dO | L log2 e | -D], each
    // 256-byte aligned: every read of a tile is a per-tile lane base (with the
    // array's address folded in) XOR a constant, plus an immediate offset
    // below 64 KiB.
    constexpr int kBuf = 2 * kTile + 2 * BR * 4;
    static_assert(kBuf % 256 == 0, "tile arrays keep the 256-byte alignment the swizzle needs");
    // 128-row tiles at d = 128 leave room for two buffers only: each tile's
    // copies are then issued in its first slots, into the buffer the previous
    // tile released, and waited for at its end.
    constexpr int NBUF = 3 * kBuf > 160 * 1024 ? 2 : 3;
    __shared__ __attribute__((aligned(256))) char Ta0[kBuf], Ta1[kBuf], Ta2[NBUF == 3 ? kBuf : 256];
    FA2_LDS char* const T0 = (FA2_LDS char*)Ta0;
    FA2_LDS char* const T1 = (FA2_LDS char*)Ta1;
    FA2_LDS char* const T2 = (FA2_LDS char*)Ta2;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int li = lane & 31;

    // Persistent workgroups: items (key tile, batch, K/V head) in order of
    // decreasing work (causal: the first key tiles have the most query tiles),
    // dealt to the workgroups in rounds, every other round in reverse order,
    // so that the work per workgroup evens out.  (Block-sparse launches one
    // workgroup per item, which then runs a single round.)
    const int BHk = p.B * p.Hkv;
    const int n_items = ((p.N + BC - 1) / BC) * BHk;
    for (int round = 0;; ++round) {
    const int slot = (round & 1) ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x;
    const int item = round * (int)gridDim.x + slot;
    if (item >= n_items) break;
    if (round > 0) __syncthreads();        // the previous item's LDS reads are done
    const int kvtile = item / BHk;
    const int bh = item - kvtile * BHk;
    const int b = bh / p.Hkv;
    const int hk = bh - b * p.Hkv;
    const int N = p.N;
    const int kv0 = kvtile * BC;
    const int kw0 = kv0 + 32 * wave;
    const int kv = kw0 + li;
    const size_t khead = ((size_t)b * p.Hkv + hk) * (size_t)N * D;

    el8 kf[KSD], vf[KSD];
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
        u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
        if (kv < N) {
            kx = global_load16(p.K + khead + (size_t)kv * D + 16 * ks + 8 * g);
            vx = global_load16(p.V + khead + (size_t)kv * D + 16 * ks + 8 * g);
        }
        kf[ks] = as_el8(kx);
        vf[ks] = as_el8(vx);
    }
    f32x16 dv[NBD], dk[NBD];
#pragma unroll
    for (int i = 0; i < NBD; ++i) {
        dv[i] = zero16();
        dk[i] = zero16();
    }

    // Query tiles: for each of the G query heads sharing this K/V head, the
    // 64-row tiles from the first one the causal mask lets through.  Block-
    // sparse: the tiles of the query blocks whose mask byte in this key
    // block's column is set (and, causal, that end at or below its first
    // key), compacted into an LDS list by wave 0.
    const int n_qt = (N + BR - 1) / BR;
    const int i_begin = CAUSAL ? kv0 / BR : 0;
    int n_i;
    FA2_LDS uint16_t* tl = nullptr;
    if constexpr (SPARSE) {
        static_assert(BC == kSparseBlock && 2 * BR == kSparseBlock, "one mask column, two query tiles per block");
        __shared__ uint16_t tl_arr[kSparseMaxN / BR];
        __shared__ int tl_count;
        tl = (FA2_LDS uint16_t*)tl_arr;
        if (wave == 0) {
            const int nb = p.nb;
            const int n = build_tile_list(tl, nb, n_qt, lane, [&](int r) {
                return p.bmask[(size_t)r * nb + kvtile] != 0 && (!CAUSAL || r >= kvtile) ? 1 : 0;
            });
            if (lane == 0) tl_count = n;
        }
        __syncthreads();
        n_i = __builtin_amdgcn_readfirstlane(tl_count);
    } else {
        n_i = n_qt - i_begin;
    }
    const int n_iter = n_i * p.G;
    // First row of query tile i of the walk.
    auto qrow_at = [&](int i) -> int {
        if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)(tl[i] & 0xfff)) * BR;
        else return (i_begin + i) * BR;
    };

    // Copy of query tile `it` into LDS as NCOPY wave instructions, which the
    // tile program spreads over the slots of its last phase: Q and dO rows
    // (clamped to N-1 past the end; those rows have L = +inf, so P = dS = 0),
    // and the padded L log2 e and -D rows (waves 0 and 2 both copy L, 1 and 3
    // both copy -D: identical bytes, so every wave issues the same number of
    // copies).
    constexpr int NCOPY = 2 * PERW + 1;
    struct TileCopy {
        const char* qbase;
        const char* obase;
        const float* ld_src;
        int last, lr, lc;
        FA2_LDS char* T;
    };
    auto plan_copy = [&](int it, FA2_LDS char* T) {
        const int hq = hk * p.G + it / n_i;
        const int qt0 = qrow_at(it % n_i);
        const size_t qrow0 = ((size_t)b * p.Hq + hq) * (size_t)N + qt0;
        const size_t prow = ((size_t)b * p.Hq + hq) * (size_t)p.Npad + qt0;
        TileCopy c;
        c.qbase = reinterpret_cast<const char*>(p.Q + qrow0 * D);
        c.obase = reinterpret_cast<const char*>(p.dO + qrow0 * D);
        c.ld_src = (wave & 1) ? p.Dneg + prow : p.L2 + prow;
        c.last = N - 1 - qt0;
        c.lr = lane / CPR;
        c.lc = 16 * ((lane % CPR) ^ swz<RB>(lane / CPR));
        asm volatile("" : "+v"(c.lr), "+v"(c.lc));   // rebuilt per tile instead of held across the loop
        c.T = T;
        return c;
    };
    auto copy_part = [&](const TileCopy& c, int j) {
        if (j < 2 * PERW) {
            const int i = j % PERW;
            const int R = (wave * PERW + i) * RPI;
            const uint32_t off = (uint32_t)(min(R + c.lr, c.last) * RB + (c.lc ^ (16 * swz<RB>(R))));
            if (j < PERW) copy_to_lds16(c.qbase, off, c.T + (wave * PERW + i) * 1024);
            else copy_to_lds16(c.obase, off, c.T + kTile + (wave * PERW + i) * 1024);
        } else {
            // 64 rows per instruction: with 128-row tiles waves 0, 2 copy the
            // two halves of L, waves 1, 3 those of -D.
            const int lh = BR == 128 ? wave >> 1 : 0;
            copy_to_lds4(c.ld_src + 64 * lh, 4 * lane, c.T + 2 * kTile + (wave & 1) * BR * 4 + 256 * lh);
        }
    };
    auto copy_tile = [&](int it, FA2_LDS char* T) {
        const TileCopy c = plan_copy(it, T);
#pragma unroll
        for (int j = 0; j < NCOPY; ++j) copy_part(c, j);
    };

    // LDS operand addresses: the swizzle only flips bits 4.. of a row's byte
    // offset below RB, so they are a per-lane base XOR a constant (32*ks for
    // Q / dO rows, chunk 2*ks + g; 64*db for the transposed reads).
    const int j16 = lane & 15;
    const int xq = 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1);
    const int r1 = 4 * g + (j16 >> 2), r2 = r1 + 8;
    const int kb_lane = li * RB + 16 * (g ^ swz<RB>(li));
    const int vb1_lane = r1 * RB + 8 * (j16 & 1) + 16 * (xq ^ swz<RB>(r1));
    const int vb2_lane = r2 * RB + 8 * (j16 & 1) + 16 * (xq ^ swz<RB>(r2));

    // One query tile as a fixed program of matrix products, one per slot
    // (NS = 2 * D/16 products of s and dp per 32-row block, NG = 4 * D/32 of
    // dV and dK; 16, 16 for d = 128):
    //   s, dp of block 0          (A: Q / dO rows, B: K / V of this lane)
    //   s, dp of block 1          | P, dS of block 0, 16 / NS elements per slot
    //   ...
    //   s, dp of block NB-1       | P, dS of block NB-2
    //   dV, dK over block 0       | P, dS of block NB-1, 16 / NG elements per slot
    //   dV, dK over blocks 1 .. NB-1
    // Each product's A operand is read from LDS kPrefetch slots ahead; a
    // scheduling fence between slots keeps this order, so the compiler waits
    // only for the read a product needs.  A block's scores live from its s, dp
    // products to the end of its P, dS (two slots into block b+2's products),
    // hence three score buffers.
    constexpr int NS = 2 * KSD, NG = 4 * NBD, NP = NB * NS + NB * NG;
    constexpr int kPrefetch = 4;
    static_assert(16 % NS == 0 && 16 % NG == 0 && NS >= 8, "slot program shape");
    static_assert(NCOPY <= NB * NG, "the copies of the next tile fit in the dV, dK phases");
    // The next tile's copies take the last slots of the last dV, dK phase (and
    // of the one before it when they do not fit).
    constexpr int kCopy0 = NBUF == 2 ? 0 : NB * NS + (NB - 1) * NG - (NCOPY > NG ? NCOPY - NG : 0);
    constexpr int NSB = NB > 2 ? 3 : 2;       // score buffers
    auto tile = [&](const FA2_LDS char* T, int qt0, const TileCopy& cp) {
        // Lane bases with the tile's address folded in, rebuilt per tile (opaque
        // to the compiler) rather than held across the loop.
        const uint32_t tb = (uint32_t)(uintptr_t)T;
        uint32_t kb = tb + kb_lane, vb1 = tb + vb1_lane, vb2 = tb + vb2_lane, lb = tb + 2 * kTile + 16 * g;
        asm volatile("" : "+v"(kb), "+v"(vb1), "+v"(vb2), "+v"(lb));
        auto at = [](uint32_t a) { return (const FA2_LDS char*)(uintptr_t)a; };
        // Four consecutive floats of the L log2 e (which = 0) or -D (which = 1)
        // rows: queries 32 * blk + 8 * rl + 4g .. +3, the order of a score
        // accumulator's registers 4 rl .. 4 rl + 3.
        auto ld_rows = [&](int which, int blk, int rl) {
            return *reinterpret_cast<const FA2_LDS f32x4*>(at(lb) + 4 * (which * BR + 32 * blk + 8 * rl));
        };
        f32x16 sc[NSB], dpc[NSB];            // block b's scores in buffer b % NSB
        uint32_t pp[NB][8], pd[NB][8];
        f32x4 lv[2][4];                      // block b's L in buffer b % 2
        f32x16 nd[2];                        // -D of block b (buffer b % 2): where its dP products start
        auto load_nd = [&](int blk, int rl) {
            const f32x4 v = ld_rows(1, blk, rl);
#pragma unroll
            for (int e = 0; e < 4; ++e) nd[blk % 2][4 * rl + e] = v[e];
        };
        // A operand of product k.
        auto load_a = [&](int k) -> el8 {
            if (k < NB * NS) {
                const int blk = k / NS, ks = (k % NS) >> 1;
                const int off = ((k & 1) ? kTile : 0) + 32 * blk * RB;          // dO or Q rows
                return as_el8(lds_load16(at(kb ^ (32 * ks)) + off));
            }
            const int j = k - NB * NS, blk = j / NG, jj = j % NG, h = jj / (NG / 2), db = (jj % (NG / 2)) >> 1;
            const int off = ((jj & 1) ? 0 : kTile) + 16 * (2 * blk + h) * RB;   // Q or dO, transposed
            return cat_tr(lds_load_tr(at(vb1 ^ (64 * db)) + off), lds_load_tr(at(vb2 ^ (64 * db)) + off));
        };
        auto product = [&](int k, el8 a) {
            if (k < NB * NS) {
                const int blk = k / NS, ks = (k % NS) >> 1, sb = blk % NSB;
                if (k & 1) dpc[sb] = mfma32(a, vf[ks], ks == 0 ? nd[blk % 2] : dpc[sb]);   // dp - D
                else sc[sb] = mfma32(a, kf[ks], ks == 0 ? zero16() : sc[sb]);
                return;
            }
            const int j = k - NB * NS, blk = j / NG, jj = j % NG, h = jj / (NG / 2), db = (jj % (NG / 2)) >> 1;
            if (jj & 1) {
                const el8 bs = as_el8(u32x4{pd[blk][4 * h], pd[blk][4 * h + 1], pd[blk][4 * h + 2], pd[blk][4 * h + 3]});
                dk[db] = mfma32(a, bs, dk[db]);
            } else {
                const el8 bp = as_el8(u32x4{pp[blk][4 * h], pp[blk][4 * h + 1], pp[blk][4 * h + 2], pp[blk][4 * h + 3]});
                dv[db] = mfma32(a, bp, dv[db]);
            }
        };
        // Element r of P and dS of block blk (query 8*(r/4) + 4g + r%4 of the
        // block, this lane's key) in three stages -- c*s - L log2 e, exp2, then
        // dS and the bf16 packing -- run for elements r, r-1, r-2 in one slot,
        // so the instructions of a slot do not wait on each other.
        // Each stage's result is pinned in its slot (an empty asm that redefines
        // it), or the compiler sinks the arithmetic down to the dV / dK products
        // that consume it and the slots before those get no vector work.
        auto pin = [](float& x) { asm volatile("" : "+v"(x)); };
        auto pin_u = [](uint32_t& x) { asm volatile("" : "+v"(x)); };
        auto stage_a = [&](int blk, int r) {
            float x = fmaf(sc[blk % NSB][r], p.c, -lv[blk % 2][r >> 2][r & 3]);
            pin(x);
            sc[blk % NSB][r] = x;
        };
        auto stage_b = [&](int blk, int r) {
            float x = exp2_fast(sc[blk % NSB][r]);
            pin(x);
            sc[blk % NSB][r] = x;
        };
        auto stage_c = [&](int blk, int r) {
            const int sb = blk % NSB;
            const float pr = sc[sb][r];
            float ds = pr * dpc[sb][r];
            pin(ds);
            dpc[sb][r] = ds;                 // the fp32 values are kept until their pair is packed
            if (r & 1) {
                uint32_t a = pack_el(sc[sb][r - 1], pr), c = pack_el(dpc[sb][r - 1], ds);
                pin_u(a);
                pin_u(c);
                pp[blk][r >> 1] = a;
                pd[blk][r >> 1] = c;
            }
        };
        // Vector work of slot k: L of block b is read in slots b*NS + NS/2 ..
        // +3, half a block of products before its P, with -D of block b + 1;
        // then the staged elements.
        auto vector_work = [&](int k) {
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
                const int rl = k - (blk * NS + NS / 2);
                if (rl >= 0 && rl < 4) {
                    lv[blk % 2][rl] = ld_rows(0, blk, rl);
                    if (blk + 1 < NB) load_nd(blk + 1, rl);
                }
            }
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
                const bool last = blk == NB - 1;
                const int start = last ? NB * NS : (blk + 1) * NS;   // first slot of the block's elements
                const int E = 16 / (last ? NG : NS);                 // elements per slot
                const int t = k - start;
#pragma unroll
                for (int i = 0; i < E; ++i) {
                    const int ra = t * E + i, rb = (t - 1) * E + i, rc = (t - 2) * E + i;
                    if (rc >= 0 && rc < 16) stage_c(blk, rc);
                    if (rb >= 0 && rb < 16) stage_b(blk, rb);
                    if (ra >= 0 && ra < 16) stage_a(blk, ra);
                }
            }
        };
        // Causal mask of block blk, once its scores are complete: only a block
        // that starts below this wave's last key has keys above the diagonal
        // (one or two blocks per query head in a wave's whole loop).
        auto mask = [&](int blk) {
            if (CAUSAL && qt0 + 32 * blk < kw0 + 31) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (kv > qt0 + 32 * blk + 8 * (i >> 2) + 4 * g + (i & 3)) sc[blk % NSB][i] = -kInf;
            }
        };
        // -D of block 0 before the first operands: its dP products start at slot 1.
#pragma unroll
        for (int rl = 0; rl < 4; ++rl) load_nd(0, rl);
        el8 abuf[kPrefetch];
        auto slot = [&](int k) {
            __builtin_amdgcn_sched_barrier(0);
            const el8 a = abuf[k % kPrefetch];
            if (k + kPrefetch < NP) abuf[k % kPrefetch] = load_a(k + kPrefetch);
            product(k, a);
            vector_work(k);
            const int jc = k - kCopy0;                      // the next tile's copies
            if (jc >= 0 && jc < NCOPY) copy_part(cp, jc);
        };
#pragma unroll
        for (int k = 0; k < kPrefetch; ++k) abuf[k] = load_a(k);
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
#pragma unroll
            for (int k = blk * NS; k < (blk + 1) * NS; ++k) slot(k);
            mask(blk);
        }
        // At d = 64 two workgroups share a CU: the dV, dK phase runs at raised
        // wave priority (3-4 % on the K/V loop; priority on the s, dp phase
        // instead gained 0-3 %).
        if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int k = NB * NS; k < NP; ++k) slot(k);
        if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
    };

    auto step = [&](int it, const FA2_LDS char* T, FA2_LDS char* Tw) __attribute__((always_inline)) {
        // Copies past the last tile repeat it into a released buffer that is
        // never read, so every step issues and waits for the same count.
        tile(T, qrow_at(it % n_i), plan_copy(min(it + NBUF - 1, n_iter - 1), Tw));
        if constexpr (NBUF == 3) wait_vm_keep<NCOPY>();   // tile it+1, issued one step earlier, has landed
        else wait_vm_all();                                // tile it+1, issued at this step's start
        barrier_lds();
    };

    if (n_iter > 0) {
        copy_tile(0, T0);
        if (NBUF == 3 && n_iter > 1) copy_tile(1, T1);
        wait_vm_all();
        __syncthreads();
        if constexpr (NBUF == 3) {
            for (int it = 0; it < n_iter; it += 3) {
                step(it, T0, T2);
                if (it + 1 < n_iter) {
                    step(it + 1, T1, T0);
                    if (it + 2 < n_iter) step(it + 2, T2, T1);
                }
            }
        } else {
            for (int it = 0; it < n_iter; it += 2) {
                step(it, T0, T1);
                if (it + 1 < n_iter) step(it + 1, T1, T0);
            }
        }
        wait_vm_all();
    }

    // epilogue: this lane's key, the whole head dim
    if (kv < N) {
        uint16_t* dVr = p.dV + khead + (size_t)kv * D;
        uint16_t* dKr = p.dK + khead + (size_t)kv * D;
#pragma unroll
        for (int db = 0; db < NBD; ++db)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int d0 = 32 * db + 8 * rq + 4 * g;
                *reinterpret_cast<u32x2*>(dVr + d0) =
                    u32x2{pack_el(dv[db][4 * rq], dv[db][4 * rq + 1]),
                          pack_el(dv[db][4 * rq + 2], dv[db][4 * rq + 3])};
                *reinterpret_cast<u32x2*>(dKr + d0) =
                    u32x2{pack_el(dk[db][4 * rq] * p.scale, dk[db][4 * rq + 1] * p.scale),
                          pack_el(dk[db][4 * rq + 2] * p.scale, dk[db][4 * rq + 3] * p.scale)};
            }
    }
    }
}

// ---------------------------------------------------------------------------------------------
// bwd_kv256f: the K/V-tile loop for d = 256 with the whole head dim of dK and
// dV in one workgroup, so s = Q K^T and dp = dO V^T are computed once per key
// tile.  Each wave owns 32 keys: their K and V rows (all 256 dims, 128 VGPRs)
// are the B operands of s and dp, and their dK and dV (32 keys x 256 dims
// each, all 256 AGPRs) accumulate from matrix products issued as inline
// assembly.  That leaves room for one 32-row query block of scores at a time,
// so query tiles have 32 rows, copied into a ring of four LDS buffers two
// tiles ahead.  A tile is a fixed program of 64 products:
//   s, dp of this tile's block         (A: Q / dO rows, B: K / V of this lane)
//   dV, dK over the previous block     | P, dS of this block, element by element
// (A: dO^T / Q^T read transposed from the previous tile's buffer, B: that
// block's P and dS, packed in registers), so the vector work of a block runs
// beside the products of the block before it; a last program without s, dp
// adds the final block.  Block-sparse (SPARSE): the key tile is one mask
// column, and the walk is the list of 32-row tiles of the query blocks its
// mask column keeps (causal: at or below the diagonal).
template <bool CAUSAL, bool SPARSE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_kv256f_kernel(const BwdParams p) {
    constexpr int D = 256;
    constexpr int NW = 4, BC = 32 * NW, BR = 32;
    constexpr int RB = 2 * D;                 // bytes per row of the Q / dO tiles
    constexpr int kTile = BR * RB;
    constexpr int KSD = D / 16;               // reduction steps over the head dim
    constexpr int NBD = D / 32;               // 32-wide head-dim blocks of dK / dV
    constexpr int RPI = 1024 / RB;            // tile rows per wave copy instruction
    constexpr int CPR = RB / 16;              // 16-byte chunks per row
    constexpr int PERW = kTile / 1024 / NW;   // copy instructions per wave per tensor
    static_assert(PERW >= 1 && kTile % (1024 * NW) == 0, "tile / waves mismatch");
    // L log2 e and -D travel as the kBwdRowPad-row chunk holding the tile (the
    // workspace rows are padded to whole chunks, so the copy stays in bounds).
    constexpr int LR = kBwdRowPad;
    static_assert(LR % BR == 0 && LR == 64, "one copy instruction per L / D chunk");
    constexpr int kBuf = 2 * kTile + 2 * LR * 4;
    static_assert(kBuf % 512 == 0, "tile arrays keep the 512-byte alignment the swizzle needs");
    __shared__ __attribute__((aligned(512))) char Ta0[kBuf], Ta1[kBuf], Ta2[kBuf], Ta3[kBuf];
    FA2_LDS char* const T0 = (FA2_LDS char*)Ta0;
    FA2_LDS char* const T1 = (FA2_LDS char*)Ta1;
    FA2_LDS char* const T2 = (FA2_LDS char*)Ta2;
    FA2_LDS char* const T3 = (FA2_LDS char*)Ta3;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int li = lane & 31;

    // Workgroups in order of decreasing work (causal: the first key tiles have
    // the most query tiles).
    const int BHk = p.B * p.Hkv;
    const int kvtile = blockIdx.x / BHk;
    const int bh = blockIdx.x - kvtile * BHk;
    const int b = bh / p.Hkv;
    const int hk = bh - b * p.Hkv;
    const int N = p.N;
    const int kv0 = kvtile * BC;
    const int kw0 = kv0 + 32 * wave;
    const int kv = kw0 + li;
    const size_t khead = ((size_t)b * p.Hkv + hk) * (size_t)N * D;

    el8 kf[KSD], vf[KSD];
    {
        // Rows past N repeat row N - 1: a lane's key only meets its own dK, dV
        // column, which is not stored.
        const size_t krow = khead + (size_t)min(kv, N - 1) * D;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            kf[ks] = as_el8(global_load16(p.K + krow + 16 * ks + 8 * g));
            vf[ks] = as_el8(global_load16(p.V + krow + 16 * ks + 8 * g));
        }
    }
    f32x16 dv[NBD], dk[NBD];
#pragma unroll
    for (int i = 0; i < NBD; ++i) {
        dv[i] = zero16();
        dk[i] = zero16();
    }

    // Query tiles: for each of the G query heads sharing this K/V head, the
    // 32-row tiles from the first one the causal mask lets through.
    const int n_qt = (N + BR - 1) / BR;
    const int i_begin = CAUSAL ? kv0 / BR : 0;
    int n_i;
    FA2_LDS uint16_t* tl = nullptr;
    if constexpr (SPARSE) {
        static_assert(BC == kSparseBlock && kSparseBlock % BR == 0, "one mask column per key tile");
        __shared__ uint16_t tl_arr[kSparseMaxN / BR];
        __shared__ int tl_count;
        tl = (FA2_LDS uint16_t*)tl_arr;
        if (wave == 0) {
            const int nb = p.nb;
            const int n = build_block_tiles<kSparseBlock / BR>(tl, nb, n_qt, lane, [&](int r) {
                return p.bmask[(size_t)r * nb + kvtile] != 0 && (!CAUSAL || r >= kvtile);
            });
            if (lane == 0) tl_count = n;
        }
        __syncthreads();
        n_i = __builtin_amdgcn_readfirstlane(tl_count);
    } else {
        n_i = n_qt - i_begin;
    }
    const int n_iter = n_i * p.G;
    auto qrow_at = [&](int i) -> int {
        if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)tl[i]) * BR;
        else return (i_begin + i) * BR;
    };

    // Copy of query tile `it` into LDS as NCOPY wave instructions: Q and dO
    // rows (clamped to N-1 past the end; those rows have L = +inf, so P = dS =
    // 0), and the L log2 e and -D chunk (waves 0 and 2 both copy L, 1 and 3
    // both copy -D: identical bytes, so every wave issues the same number of
    // copies).
    constexpr int NCOPY = 2 * PERW + 1;
    struct TileCopy {
        const char* qbase;
        const char* obase;
        const float* ld_src;
        int last, lr, lc;
        FA2_LDS char* T;
    };
    auto plan_copy = [&](int it, FA2_LDS char* T) {
        const int hq = hk * p.G + it / n_i;
        const int qt0 = qrow_at(it % n_i);
        const size_t qrow0 = ((size_t)b * p.Hq + hq) * (size_t)N + qt0;
        const size_t prow = ((size_t)b * p.Hq + hq) * (size_t)p.Npad + (qt0 & ~(LR - 1));
        TileCopy c;
        c.qbase = reinterpret_cast<const char*>(p.Q + qrow0 * D);
        c.obase = reinterpret_cast<const char*>(p.dO + qrow0 * D);
        c.ld_src = (wave & 1) ? p.Dneg + prow : p.L2 + prow;
        c.last = N - 1 - qt0;
        c.lr = lane / CPR;
        c.lc = 16 * ((lane % CPR) ^ swz<RB>(lane / CPR));
        asm volatile("" : "+v"(c.lr), "+v"(c.lc));   // rebuilt per tile instead of held across the loop
        c.T = T;
        return c;
    };
    auto copy_part = [&](const TileCopy& c, int j) {
        if (j < 2 * PERW) {
            const int i = j % PERW;
            const int R = (wave * PERW + i) * RPI;
            const uint32_t off = (uint32_t)(min(R + c.lr, c.last) * RB + (c.lc ^ (16 * swz<RB>(R))));
            if (j < PERW) copy_to_lds16(c.qbase, off, c.T + (wave * PERW + i) * 1024);
            else copy_to_lds16(c.obase, off, c.T + kTile + (wave * PERW + i) * 1024);
        } else {
            copy_to_lds4(c.ld_src, 4 * lane, c.T + 2 * kTile + (wave & 1) * LR * 4);
        }
    };
    auto copy_tile = [&](int it, FA2_LDS char* T) {
        const TileCopy c = plan_copy(it, T);
#pragma unroll
        for (int j = 0; j < NCOPY; ++j) copy_part(c, j);
    };

    // LDS operand addresses: per-lane bases XOR a constant (32*ks for Q / dO
    // rows, chunk 2*ks + g; 64*db for the transposed reads).
    const int j16 = lane & 15;
    const int xq = 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1);
    const int r1 = 4 * g + (j16 >> 2), r2 = r1 + 8;
    const int kb_lane = li * RB + 16 * (g ^ swz<RB>(li));
    const int vb1_lane = r1 * RB + 8 * (j16 & 1) + 16 * (xq ^ swz<RB>(r1));
    const int vb2_lane = r2 * RB + 8 * (j16 & 1) + 16 * (xq ^ swz<RB>(r2));

    constexpr int NS = 2 * KSD;               // s, dp products of a block
    constexpr int NG = 4 * NBD;               // dV, dK products of a block
    constexpr int NP = NS + NG;
    constexpr int kPrefetch = 4;
    static_assert(NCOPY < NS, "the copies of a tile fit in the first phase");
    uint32_t qp[8], qd[8];                    // P, dS of the previous block, packed
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        qp[r] = 0u;
        qd[r] = 0u;
    }
    // Tile program; with DRAIN only the dV, dK products of the previous block.
    auto tile = [&](auto drain_tag, const FA2_LDS char* T, const FA2_LDS char* Tp, int qt0,
                    const TileCopy& cp) __attribute__((always_inline)) {
        constexpr bool DRAIN = decltype(drain_tag)::value;
        const uint32_t tb = (uint32_t)(uintptr_t)T, tp = (uint32_t)(uintptr_t)Tp;
        uint32_t kb = tb + kb_lane, vb1 = tp + vb1_lane, vb2 = tp + vb2_lane;
        uint32_t lb = tb + 2 * kTile + 16 * g + 4 * (qt0 & (LR - 1));
        asm volatile("" : "+v"(kb), "+v"(vb1), "+v"(vb2), "+v"(lb));
        auto at = [](uint32_t a) { return (const FA2_LDS char*)(uintptr_t)a; };
        // Four consecutive floats of the L log2 e (which = 0) or -D (which = 1)
        // rows of this block: queries 8 * rl + 4g .. +3, the order of a score
        // accumulator's registers 4 rl .. 4 rl + 3.
        auto ld_rows = [&](int which, int rl) {
            return *reinterpret_cast<const FA2_LDS f32x4*>(at(lb) + 4 * (which * LR + 8 * rl));
        };
        f32x16 sc, dpc, nd;
        f32x4 lv[4];
        uint32_t pp[8], pd[8];
        auto load_a = [&](int k) -> el8 {
            if (k < NS) {
                const int ks = k >> 1;
                return as_el8(lds_load16(at(kb ^ (32 * ks)) + ((k & 1) ? kTile : 0)));   // dO or Q rows
            }
            const int j = k - NS, h = j >> 4, db = (j & 15) >> 1;
            const int off = ((j & 1) ? 0 : kTile) + 16 * h * RB;                      // Q or dO, transposed
            return cat_tr(lds_load_tr(at(vb1 ^ (64 * db)) + off), lds_load_tr(at(vb2 ^ (64 * db)) + off));
        };
        auto product = [&](int k, el8 a) {
            if (k < NS) {
                const int ks = k >> 1;
                if (k & 1) dpc = mfma32(a, vf[ks], ks == 0 ? nd : dpc);                 // dp - D
                else sc = mfma32(a, kf[ks], ks == 0 ? zero16() : sc);
                return;
            }
            const int j = k - NS, h = j >> 4, db = (j & 15) >> 1;
            // Issued as assembly to keep the accumulators in AGPRs.
            if (j & 1) {
                const el8 bs = as_el8(u32x4{qd[4 * h], qd[4 * h + 1], qd[4 * h + 2], qd[4 * h + 3]});
                f32x16 c = dk[db];
                asm volatile(FA2_MFMA_32X32X16 " %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(bs));
                dk[db] = c;
            } else {
                const el8 bp = as_el8(u32x4{qp[4 * h], qp[4 * h + 1], qp[4 * h + 2], qp[4 * h + 3]});
                f32x16 c = dv[db];
                asm volatile(FA2_MFMA_32X32X16 " %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(bp));
                dv[db] = c;
            }
        };
        // Element r of P and dS (query 8*(r/4) + 4g + r%4 of the block, this
        // lane's key) in three stages -- c*s - L log2 e, exp2, then dS and the
        // bf16 packing -- each pinned in its slot.
        auto pin = [](float& x) { asm volatile("" : "+v"(x)); };
        auto pin_u = [](uint32_t& x) { asm volatile("" : "+v"(x)); };
        auto stage_a = [&](int r) {
            float x = fmaf(sc[r], p.c, -lv[r >> 2][r & 3]);
            pin(x);
            sc[r] = x;
        };
        auto stage_b = [&](int r) {
            float x = exp2_fast(sc[r]);
            pin(x);
            sc[r] = x;
        };
        auto stage_c = [&](int r) {
            const float pr = sc[r];
            float ds = pr * dpc[r];
            pin(ds);
            dpc[r] = ds;
            if (r & 1) {
                uint32_t a = pack_el(sc[r - 1], pr), c = pack_el(dpc[r - 1], ds);
                pin_u(a);
                pin_u(c);
                pp[r >> 1] = a;
                pd[r >> 1] = c;
            }
        };
        auto vector_work = [&](int k) {
            if constexpr (!DRAIN) {
                const int rl = k - NS / 2;                    // L of the block, half a phase ahead
                if (rl >= 0 && rl < 4) lv[rl] = ld_rows(0, rl);
#pragma unroll
                for (int r = 0; r < 16; ++r) {                // element r starts at slot NS + r * (NG - 3) / 15
                    const int t = k - NS - r * (NG - 3) / 15;
                    if (t == 2) stage_c(r);
                    if (t == 1) stage_b(r);
                    if (t == 0) stage_a(r);
                }
            }
        };
        if constexpr (!DRAIN) {
#pragma unroll
            for (int rl = 0; rl < 4; ++rl) {                  // -D: where the dP products start
                const f32x4 v = ld_rows(1, rl);
#pragma unroll
                for (int e = 0; e < 4; ++e) nd[4 * rl + e] = v[e];
            }
        }
        constexpr int K0 = DRAIN ? NS : 0;
        el8 abuf[kPrefetch];
        auto slot = [&](int k) {
            __builtin_amdgcn_sched_barrier(0);
            const el8 a = abuf[k % kPrefetch];
            if (k + kPrefetch < NP) abuf[k % kPrefetch] = load_a(k + kPrefetch);
            product(k, a);
            vector_work(k);
            if (!DRAIN && k >= 1 && k <= NCOPY) copy_part(cp, k - 1);
        };
#pragma unroll
        for (int k = K0; k < K0 + kPrefetch; ++k) abuf[k % kPrefetch] = load_a(k);
        if constexpr (!DRAIN) {
#pragma unroll
            for (int k = 0; k < NS; ++k) slot(k);
            // Causal mask, once the scores are complete: only a block that starts
            // below this wave's last key has keys above the diagonal.
            if (CAUSAL && qt0 < kw0 + 31) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (kv > qt0 + 8 * (i >> 2) + 4 * g + (i & 3)) sc[i] = -kInf;
            }
        }
#pragma unroll
        for (int k = NS; k < NP; ++k) slot(k);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!DRAIN) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                qp[r] = pp[r];
                qd[r] = pd[r];
            }
        }
    };

    // Step it reads tile it (and the previous tile's buffer) and copies tile
    // it + 2 into the buffer released by the barrier ending step it - 1;
    // copies past the last tile repeat it into a buffer never read, so every
    // step issues and waits for the same count.
    auto step = [&](int it, const FA2_LDS char* T, const FA2_LDS char* Tp, FA2_LDS char* Tw)
        __attribute__((always_inline)) {
        tile(std::false_type{}, T, Tp, qrow_at(it % n_i), plan_copy(min(it + 2, n_iter - 1), Tw));
        wait_vm_keep<NCOPY>();          // tile it+1, issued one step earlier, has landed
        barrier_lds();
    };

    if (n_iter > 0) {
        // Tile -1 (the previous buffer of tile 0): zero Q and dO, so the first
        // dV, dK products add nothing.
        for (int i = tid; i < 2 * kTile / 16; i += 64 * NW) lds_store16(T3 + 16 * i, u32x4{0, 0, 0, 0});
        copy_tile(0, T0);
        copy_tile(min(1, n_iter - 1), T1);
        wait_vm_all();
        __syncthreads();
        for (int it = 0; it < n_iter; it += 4) {
            step(it, T0, T3, T2);
            if (it + 1 < n_iter) {
                step(it + 1, T1, T0, T3);
                if (it + 2 < n_iter) {
                    step(it + 2, T2, T1, T0);
                    if (it + 3 < n_iter) step(it + 3, T3, T2, T1);
                }
            }
        }
        // The last block's dV, dK, from the last tile's buffer.
        const int t = (n_iter - 1) & 3;
        const FA2_LDS char* Tl = t == 0 ? T0 : t == 1 ? T1 : t == 2 ? T2 : T3;
        tile(std::true_type{}, Tl, Tl, 0, plan_copy(0, T0));
        wait_vm_all();
    }
    // The accumulators were last written by matrix products issued from inline
    // assembly, which the compiler does not track: wait them out before reading.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    // epilogue: this lane's key, the whole head dim
    if (kv < N) {
        uint16_t* dVr = p.dV + khead + (size_t)kv * D;
        uint16_t* dKr = p.dK + khead + (size_t)kv * D;
#pragma unroll
        for (int db = 0; db < NBD; ++db)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int d0 = 32 * db + 8 * rq + 4 * g;
                *reinterpret_cast<u32x2*>(dVr + d0) =
                    u32x2{pack_el(dv[db][4 * rq], dv[db][4 * rq + 1]),
                          pack_el(dv[db][4 * rq + 2], dv[db][4 * rq + 3])};
                *reinterpret_cast<u32x2*>(dKr + d0) =
                    u32x2{pack_el(dk[db][4 * rq] * p.scale, dk[db][4 * rq + 1] * p.scale),
                          pack_el(dk[db][4 * rq + 2] * p.scale, dk[db][4 * rq + 3] * p.scale)};
            }
    }
}

// ---------------------------------------------------------------------------------------------
// dQ = bf16(scale * accumulator), 8 elements per thread.
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(const BwdParams p, long n8) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const float* src = p.dQacc + i * 8;
    const u32x4 a = *reinterpret_cast<const u32x4*>(src);
    const u32x4 c = *reinterpret_cast<const u32x4*>(src + 4);
    u32x4 out;
    out[0] = pack_el(u32_as_f32(a[0]) * p.scale, u32_as_f32(a[1]) * p.scale);
    out[1] = pack_el(u32_as_f32(a[2]) * p.scale, u32_as_f32(a[3]) * p.scale);
    out[2] = pack_el(u32_as_f32(c[0]) * p.scale, u32_as_f32(c[1]) * p.scale);
    out[3] = pack_el(u32_as_f32(c[2]) * p.scale, u32_as_f32(c[3]) * p.scale);
    *reinterpret_cast<u32x4*>(p.dQ + i * 8) = out;
}

// Workgroups of a persistent launch: per_cu resident workgroups on every
// compute unit of the current device (the count is read once per device).
long persistent_workgroups(int per_cu) {
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256L * per_cu;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return (long)cus[dev] * per_cu;
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdParams& p, unsigned stages, hipStream_t stream) {
    BwdParams arg = p;
    const long rows = (long)p.B * p.Hq * p.N;
    const long rows_pad = (long)p.B * p.Hq * p.Npad;
    const bool atomic_dq = (stages & 8u) != 0;
    if (p.bmask && atomic_dq) return hipErrorInvalidValue;   // block-sparse: dQ in its own pass
    if (stages & 1u) {
        constexpr int RPB = 256 / (D / 8);
        long rows_arg = rows_pad;
        int zero = atomic_dq ? 1 : 0;
        void* args[] = {&arg, &rows_arg, &zero};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_pre_kernel<D>),
                                       dim3((unsigned)((rows_pad + RPB - 1) / RPB)), dim3(256), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    if (stages & 2u) {
        void* args[] = {&arg};
        const void* fn;
        long grid;
        unsigned threads;
        if constexpr (D <= 128) {
            if (atomic_dq) {
                fn = reinterpret_cast<const void*>(&bwd_pair_kernel<D, CAUSAL, true>);
                threads = 512;
            } else {
                // 128-row query tiles when every tile lies below N, at d = 64 and
                // for causal d = 128 (non-causal d = 128 ran slower with them).
                if (p.bmask) fn = reinterpret_cast<const void*>(&bwd_kv_kernel<D, CAUSAL, true, 2>);
                else if (D == 128 && CAUSAL && p.N % 128 == 0)
                    fn = reinterpret_cast<const void*>(&bwd_kv_kernel<D, CAUSAL, false, D == 128 && CAUSAL ? 4 : 2>);
                else fn = reinterpret_cast<const void*>(&bwd_kv_kernel<D, CAUSAL, false, 2>);
                threads = 256;
            }
            grid = (long)p.B * p.Hkv * ((p.N + 127) / 128);
            // Dense: persistent workgroups dealt the items in decreasing-work
            // order.  Block-sparse: one workgroup per item, since a mask's
            // column weights need not fall with the key tile (a local + global
            // mask's first column holds every row): 9-12 % faster there.
            if (!atomic_dq && !p.bmask) grid = std::min<long>(grid, persistent_workgroups(D == 64 ? 2 : 1));
        } else if (atomic_dq) {
            fn = reinterpret_cast<const void*>(&bwd_main_kernel<D, CAUSAL, true>);
            constexpr int BC = BwdCfg<D>::BC;
            grid = (long)p.B * p.Hkv * ((p.N + BC - 1) / BC);
            threads = 64 * BwdCfg<D>::NW;
        } else {
            fn = p.bmask ? reinterpret_cast<const void*>(&bwd_kv256f_kernel<CAUSAL, true>)
                         : reinterpret_cast<const void*>(&bwd_kv256f_kernel<CAUSAL, false>);
            grid = (long)p.B * p.Hkv * ((p.N + 127) / 128);
            threads = 256;
        }
        hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(threads), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    if (stages & 4u) {
        if (atomic_dq) {
            long n8 = rows * D / 8;
            void* args[] = {&arg, &n8};
            return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_convert_kernel),
                                   dim3((unsigned)((n8 + 255) / 256)), dim3(256), args, 0, stream);
        }
        void* args[] = {&arg};
        const int rows_per_wg = D == 128 && !p.bmask ? 256 : 128;   // block-sparse: one mask row
        const long grid = (long)p.B * p.Hq * ((p.N + rows_per_wg - 1) / rows_per_wg);
        const void* fn;
        if constexpr (D <= 128)
            fn = p.bmask ? reinterpret_cast<const void*>(&bwd_dq_pipe_kernel<D, CAUSAL, true>)
                         : reinterpret_cast<const void*>(&bwd_dq_pipe_kernel<D, CAUSAL, false>);
        else fn = p.bmask ? reinterpret_cast<const void*>(&bwd_dq256_kernel<CAUSAL, true>)
                          : reinterpret_cast<const void*>(&bwd_dq256_kernel<CAUSAL, false>);
        return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, stream);
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int d, bool causal, unsigned stages, hipStream_t stream) {
    switch (d) {
        case 64: return causal ? launch_bwd_t<64, true>(p, stages, stream) : launch_bwd_t<64, false>(p, stages, stream);
        case 128: return causal ? launch_bwd_t<128, true>(p, stages, stream) : launch_bwd_t<128, false>(p, stages, stream);
        case 256: return causal ? launch_bwd_t<256, true>(p, stages, stream) : launch_bwd_t<256, false>(p, stages, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace FA2_NS
