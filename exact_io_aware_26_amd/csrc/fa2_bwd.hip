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
// Three kernels on one stream:
//   bwd_pre        D = rowsum(dO o O) in fp32, and zeroes the fp32 dQ accumulator.
//   bwd_main       per K/V tile: dK, dV in VGPRs for the whole loop; dQ by atomics.
//   bwd_dq_convert dQ = bf16(scale * accumulator).
//
// gfx950 mapping of bwd_main (NW wave64s; each wave owns 32 keys of the tile,
// the backward analogue of splitting Q across waves):
//   * S = Q K_w^T and dP = dO V_w^T on v_mfma_f32_32x32x16_bf16 with the
//     wave's K_w / V_w rows as the B operand: every accumulator register then
//     holds one key per lane and 16 query rows, so P, dS and both gradient
//     accumulators share one register layout and need no data movement.
//   * dV^T += dO^T P and dK^T += Q^T dS take P and dS straight from registers
//     (as bf16) and read dO^T / Q^T fragments with ds_read_b64_tr_b16 from
//     row-major LDS tiles.
//   * dQ needs dS with the queries across lanes, so each wave writes its dS^T
//     block to LDS; after one barrier the waves split the dQ tile, each
//     reducing over all keys of the workgroup (dS and K both by transposed
//     LDS reads) and adding its fp32 result into the accumulator with
//     global atomics (one per element per K/V tile).
//   * LDS tiles use one XOR swizzle of the 16-byte chunks that is free of
//     bank conflicts both for 16-byte row reads (MFMA operands) and for the
//     transposed reads.
#include "fa2_device.h"
#include "fa2_kernels.h"

namespace fa2 {

namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kInf = __builtin_huge_valf();

// Swizzle of the 16-byte chunk index of an LDS row holding RB bytes.  Rows
// are read either as 8 consecutive rows x 32 bytes (MFMA row operands) or as
// 8 consecutive rows x 64 bytes (transposed reads); both hit distinct banks.
// (Rows of 64 bytes need none: four consecutive rows already span all banks.)
template <int RB> __device__ __forceinline__ int swz(int row) {
    return RB == 64 ? 0
         : RB == 128 ? 4 * ((row >> 1) & 1) + 2 * ((row >> 2) & 1)
                     : 4 * (row & 3) + 2 * ((row >> 2) & 1);
}

// Byte offset of element `col` (bf16) in row `row` of a swizzled tile with RB bytes per row.
template <int RB> __device__ __forceinline__ int tile_off(int row, int col) {
    return row * RB + 16 * ((col >> 3) ^ swz<RB>(row)) + 2 * (col & 7);
}

// A 32x16 (or 16x32) MFMA operand whose reduction index runs along the rows
// of a row-major LDS tile: two transposed reads (rows r0.. and r0+8..).
template <int RB>
__device__ __forceinline__ bf16x8 tr_operand(const FA2_LDS char* tile, int r0, int c0, int lane) {
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
__device__ __forceinline__ bf16x8 row_operand(const FA2_LDS char* tile, int r0, int c0, int lane) {
    const int row = r0 + (lane & 31);
    const int col = c0 + 8 * (lane >> 5);
    return as_bf16x8(lds_load16(tile + tile_off<RB>(row, col)));
}

// BC keys per workgroup (32 per wave), BR query rows per inner tile; K_w/V_w
// MFMA operands live in VGPRs (KV_REGS) or are re-read from LDS.
template <int D> struct BwdCfg;
template <> struct BwdCfg<64> { static constexpr int BC = 128, NW = 4, BR = 64; static constexpr bool KV_REGS = true; };
template <> struct BwdCfg<128> { static constexpr int BC = 128, NW = 4, BR = 64; static constexpr bool KV_REGS = true; };
template <> struct BwdCfg<256> { static constexpr int BC = 64, NW = 2, BR = 32; static constexpr bool KV_REGS = false; };

// ---------------------------------------------------------------------------------------------
// bwd_pre: D_i = sum_d dO_id * O_id (fp32) and zero the dQ accumulator row.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const BwdParams p, long rows) {
    constexpr int LPR = D / 8;                 // lanes per row (8 bf16 each)
    constexpr int RPB = 256 / LPR;             // rows per block
    const long row = (long)blockIdx.x * RPB + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const size_t off = (size_t)row * D + part * 8;
        const u32x4 a = global_load16(p.dO + off);
        const u32x4 b = global_load16(p.O + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t x = a[i], y = b[i];
            acc = fmaf(u32_as_f32(x << 16), u32_as_f32(y << 16), acc);
            acc = fmaf(u32_as_f32(x & 0xffff0000u), u32_as_f32(y & 0xffff0000u), acc);
        }
        float* z = p.dQacc + off;
        *reinterpret_cast<u32x4*>(z) = u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(z + 4) = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
    if (row < rows && part == 0) p.Dsum[row] = acc;
}

// ---------------------------------------------------------------------------------------------
template <int D, bool CAUSAL>
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
    constexpr int KSQ = BR / 16;       // reduction steps over the queries of a tile
    constexpr int KSKV = BC / 16;      // reduction steps over the keys of the workgroup
    constexpr int kKBytes = BC * RB_D;
    constexpr int kVBytes = KV_REGS ? 0 : BC * RB_D;
    constexpr int kQBytes = BR * RB_D;
    constexpr int kSBytes = BC * RB_Q;
    __shared__ __attribute__((aligned(16))) char smem_raw[kKBytes + kVBytes + 2 * kQBytes + kSBytes + 2 * BR * 4];
    FA2_LDS char* Ks = (FA2_LDS char*)smem_raw;
    FA2_LDS char* Vs = Ks + kKBytes;
    FA2_LDS char* Qs = Vs + kVBytes;
    FA2_LDS char* dOs = Qs + kQBytes;
    FA2_LDS char* dSt = dOs + kQBytes;
    FA2_LDS float* Ls = (FA2_LDS float*)(dSt + kSBytes);
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
    bf16x8 kf[KV_REGS ? KSD : 1], vf[KV_REGS ? KSD : 1];
    if (KV_REGS) {
#pragma unroll
        for (int ks = 0; ks < (KV_REGS ? KSD : 1); ++ks) {
            u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
            if (kv < N) {
                kx = global_load16(p.K + khead + (size_t)kv * D + 16 * ks + 8 * g);
                vx = global_load16(p.V + khead + (size_t)kv * D + 16 * ks + 8 * g);
            }
            kf[ks] = as_bf16x8(kx);
            vf[ks] = as_bf16x8(vx);
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
            const size_t r = ((size_t)b * p.Hq + hq) * (size_t)N + qt0 + tid;
            const bool in = qt0 + tid < N;
            sl = in ? p.L[r] * kLog2e : kInf;   // rows past the end get P = 0
            sd = in ? p.Dsum[r] : 0.f;
        }
    };

    if (PREFETCH && n_iter > 0) stage(0);

    for (int it = 0; it < n_iter; ++it) {
        const int hq = hk * p.G + it / n_i;
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
            Ls[tid] = sl;
            Dl[tid] = sd;
        }
        __syncthreads();                               // (A) tile visible
        if (PREFETCH && it + 1 < n_iter) stage(it + 1);  // next tile's loads in flight

        // 2. S, P, dP, dS for this wave's keys; dV, dK updates; dS^T -> LDS
        const bool wave_any = kw0 < N && !(CAUSAL && qt0 + BR - 1 < kw0);
        if (wave_any) {
            const bool need_mask = (CAUSAL && qt0 < kw0 + 32) || qt0 + BR > N || kw0 + 32 > N;
            uint32_t pp[NQB][8], sp[NQB][8];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                f32x16 s = zero16(), dp = zero16();
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    const bf16x8 aq = row_operand<RB_D>(Qs, 32 * qb, 16 * ks, lane);
                    const bf16x8 ao = row_operand<RB_D>(dOs, 32 * qb, 16 * ks, lane);
                    bf16x8 bk, bv;
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
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int ql = 32 * qb + 8 * rq + 4 * g;      // local query of register 4*rq
                    float lv[4], dv4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        lv[e] = Ls[ql + e];
                        dv4[e] = Dl[ql + e];
                    }
                    float pr[4], dsr[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * rq + e;
                        float pv = exp2_fast(fmaf(s[r], p.c, -lv[e]));
                        if (need_mask) {
                            const int qg = qt0 + ql + e;
                            if ((CAUSAL && kv > qg) || kv >= N) pv = 0.f;
                        }
                        pr[e] = pv;
                        dsr[e] = pv * (dp[r] - dv4[e]);
                    }
                    pp[qb][2 * rq] = pack_bf16(pr[0], pr[1]);
                    pp[qb][2 * rq + 1] = pack_bf16(pr[2], pr[3]);
                    sp[qb][2 * rq] = pack_bf16(dsr[0], dsr[1]);
                    sp[qb][2 * rq + 1] = pack_bf16(dsr[2], dsr[3]);
                    // dS^T[key][query .. query+3]
                    *reinterpret_cast<FA2_LDS u32x2*>(dSt + tile_off<RB_Q>(32 * wave + li, ql)) =
                        u32x2{sp[qb][2 * rq], sp[qb][2 * rq + 1]};
                }
            }
#pragma unroll
            for (int kk = 0; kk < KSQ; ++kk) {
                const int qb = kk >> 1, h = kk & 1;
                const bf16x8 bp = as_bf16x8(u32x4{pp[qb][4 * h], pp[qb][4 * h + 1], pp[qb][4 * h + 2], pp[qb][4 * h + 3]});
                const bf16x8 bs = as_bf16x8(u32x4{sp[qb][4 * h], sp[qb][4 * h + 1], sp[qb][4 * h + 2], sp[qb][4 * h + 3]});
#pragma unroll
                for (int db = 0; db < NBD; ++db) {
                    const bf16x8 ao = tr_operand<RB_D>(dOs, 16 * kk, 32 * db, lane);
                    dv[db] = mfma32(ao, bp, dv[db]);
                    const bf16x8 aq = tr_operand<RB_D>(Qs, 16 * kk, 32 * db, lane);
                    dk[db] = mfma32(aq, bs, dk[db]);
                }
            }
        } else {
            // no key of this wave is visible from this query tile: its dS^T rows are zero
#pragma unroll
            for (int ch = 0; ch < RB_Q / 16; ++ch)
                lds_store16(dSt + (32 * wave + li) * RB_Q + 16 * ch, u32x4{0, 0, 0, 0});
        }
        __syncthreads();                               // (B) dS^T of all waves visible

        // 3. dQ tile (BR x D): waves split the 32x32 output blocks; reduce over all BC keys.
        const size_t qrow0 = ((size_t)b * p.Hq + hq) * (size_t)N + qt0;
        for (int t = wave; t < NQB * NBD; t += NW) {
            const int qb = t / NBD, db = t % NBD;
            if (qt0 + 32 * qb >= N) continue;
            f32x16 acc = zero16();
            int kk_end = KSKV;
            if (CAUSAL) {
                // keys beyond the block's last query contribute dS = 0
                const int last_q = qt0 + 32 * qb + 31 - kv0;
                kk_end = min(KSKV, last_q / 16 + 1);
            }
            for (int kk = 0; kk < kk_end; ++kk) {
                const bf16x8 a = tr_operand<RB_Q>(dSt, 16 * kk, 32 * qb, lane);
                const bf16x8 bk = tr_operand<RB_D>(Ks, 16 * kk, 32 * db, lane);
                acc = mfma32(a, bk, acc);
            }
            const int d = 32 * db + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ql = 32 * qb + 8 * (r >> 2) + 4 * g + (r & 3);
                if (qt0 + ql < N) atomicAdd(p.dQacc + (qrow0 + ql) * D + d, acc[r]);
            }
        }
    }

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
                    u32x2{pack_bf16(dv[db][4 * rq], dv[db][4 * rq + 1]),
                          pack_bf16(dv[db][4 * rq + 2], dv[db][4 * rq + 3])};
                *reinterpret_cast<u32x2*>(dKr + d0) =
                    u32x2{pack_bf16(dk[db][4 * rq] * p.scale, dk[db][4 * rq + 1] * p.scale),
                          pack_bf16(dk[db][4 * rq + 2] * p.scale, dk[db][4 * rq + 3] * p.scale)};
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
    out[0] = pack_bf16(u32_as_f32(a[0]) * p.scale, u32_as_f32(a[1]) * p.scale);
    out[1] = pack_bf16(u32_as_f32(a[2]) * p.scale, u32_as_f32(a[3]) * p.scale);
    out[2] = pack_bf16(u32_as_f32(c[0]) * p.scale, u32_as_f32(c[1]) * p.scale);
    out[3] = pack_bf16(u32_as_f32(c[2]) * p.scale, u32_as_f32(c[3]) * p.scale);
    *reinterpret_cast<u32x4*>(p.dQ + i * 8) = out;
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdParams& p, unsigned stages, hipStream_t stream) {
    BwdParams arg = p;
    const long rows = (long)p.B * p.Hq * p.N;
    if (stages & 1u) {
        constexpr int RPB = 256 / (D / 8);
        long rows_arg = rows;
        void* args[] = {&arg, &rows_arg};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_pre_kernel<D>),
                                       dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    if (stages & 2u) {
        constexpr int BC = BwdCfg<D>::BC;
        const long grid = (long)p.B * p.Hkv * ((p.N + BC - 1) / BC);
        void* args[] = {&arg};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_main_kernel<D, CAUSAL>),
                                       dim3((unsigned)grid), dim3(64 * BwdCfg<D>::NW), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    if (stages & 4u) {
        long n8 = rows * D / 8;
        void* args[] = {&arg, &n8};
        return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_convert_kernel),
                               dim3((unsigned)((n8 + 255) / 256)), dim3(256), args, 0, stream);
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

}  // namespace fa2
