// fa2_fwd.hip -- FlashAttention-2 forward pass for gfx950.
//
// Method (FlashAttention-2 summary page, zhaifeiyue.github.io, section 2
// "Q2 method" and section 3): the outer loop is over blocks of query rows,
// one workgroup each (grid = batch x heads x query tiles); the inner loop
// streams K/V tiles.  Each wavefront owns its own slice of query rows and
// reads the shared K/V tile from LDS, so wavefronts never exchange partial
// results ("split-Q").  The softmax is online with a deferred rescale: the
// accumulator holds the unnormalized sum diag(exp(m_old - m_new)) O~ +
// exp(S - m_new) V and is divided by the row sum l once at the end; the
// only statistic written is L = m + log(l).  With a causal mask, tiles that
// lie wholly above the diagonal are skipped and only tiles that straddle it
// (or the ragged end of the sequence) are masked.
//
// gfx950 mapping (each wave64 owns 32 query rows; the kernels below give the
// workgroup shapes, tile sizes and the LDS pipeline):
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: the B operand is the wave's 32 query rows
//     (kept in VGPRs for the whole loop) and the A operand is K read from
//     LDS.  The accumulator layout then gives each lane ONE query row and 16
//     keys per 32-key block, so the row max and row sum are in-lane
//     reductions plus one v_permlane32_swap with lane l ^ 32.
//   * The output is accumulated transposed too, O^T = V^T P^T: P^T is the
//     score accumulator converted to bf16 in place (no data movement, the
//     accumulator layout IS the B-operand layout), and V^T fragments come
//     from a row-major V tile through ds_read_b64_tr_b16.  Each lane again
//     owns one query row of the output, so the rescale by exp2(m_old -
//     m_new) is a per-lane multiply, skipped when no row's maximum moved.
//   * Softmax runs in the log2 domain: c = scale * log2(e) is folded into
//     one FMA per score before v_exp_f32; the row sum is taken from the fp32
//     probabilities (before their rounding to bf16 for the PV product), so L
//     stays accurate to fp32 even for rows with few keys.
//   * LDS rows are XOR-swizzled by 16-byte chunk (no padding) so that the
//     MFMA operand reads are free of bank conflicts.
//   * Grid order: the causal query tiles with the most work run first, and
//     consecutive workgroup ids walk the heads of one query-tile level, so
//     with B*Hq a multiple of 8 all tiles of a head land on the same XCD
//     (workgroups are dealt round-robin to the 8 XCDs) and share its L2.
#include "fa2_device.h"
#include "fa2_kernels.h"

#include <type_traits>

namespace FA2_NS {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.693147180559945309f;

// XOR swizzle of the 16-byte chunk index within an LDS row (rows of 2*D bytes).
// The LDS serves 16-byte reads 16 lanes per clock and 8-byte reads 32 lanes
// per clock over 64 banks.  K rows are read as 16 consecutive rows x one chunk
// (MFMA row operands), V rows as 4 consecutive rows x 4 chunks (transposed
// reads); this pattern puts both on 64 distinct banks.
template <int D> __device__ __forceinline__ int swz(int row) {
    return D == 64 ? 4 * ((row >> 1) & 1) + ((row >> 2) & 3) : 4 * (row & 3) + ((row >> 2) & 3);
}

// Row of O from this lane's fp32 accumulators (the lane's 4 * NBD columns of
// one query row) scaled by inv, stored as bf16.  With Olo, each element's
// rounding residual x - bf16(x) (exact in fp32) is stored too, rounded to
// bf16: O + Olo then carries the fp32 value to about 16 significant bits,
// from which the backward forms D = rowsum(dO o O) without the 8-bit error of
// the stored O.
template <int NBD>
__device__ __forceinline__ void store_o_row(uint16_t* Orow, uint16_t* Olorow, const f32x16 (&o)[NBD],
                                            float inv, int g) {
#pragma unroll
    for (int db = 0; db < NBD; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const int d0 = 32 * db + 8 * rq + 4 * g;
            const float x0 = o[db][4 * rq] * inv, x1 = o[db][4 * rq + 1] * inv;
            const float x2 = o[db][4 * rq + 2] * inv, x3 = o[db][4 * rq + 3] * inv;
            const uint32_t w0 = pack_el(x0, x1), w1 = pack_el(x2, x3);
            *reinterpret_cast<u32x2*>(Orow + d0) = u32x2{w0, w1};
            if (Olorow)
                *reinterpret_cast<u32x2*>(Olorow + d0) =
                    u32x2{pack_el(x0 - lo_el_f32(w0), x1 - hi_el_f32(w0)),
                          pack_el(x2 - lo_el_f32(w1), x3 - hi_el_f32(w1))};
        }
}

// Pipelined forward for d = 64 and 128: one workgroup = 4 wave64s of 32 query
// rows each (128 rows, one mask block of block-sparse attention), with several
// workgroups resident per CU, so the waves sharing a SIMD come from
// independent workgroups and cover each other's waits and barriers: at d = 64
// three per CU (165 registers, 48 KiB of LDS; three waves per SIMD; two for
// block-sparse, with its tile list), at d = 128 two per CU (250 registers;
// two-deep K/V rings of 64 KiB).  Against one
// 8-wave, 256-row workgroup per CU this ran 2-8 % faster dense and 8-30 %
// faster block-sparse.
//   * K/V tiles are copied from global memory straight into LDS
//     (global_load_lds_dwordx4, no staging registers), K one tile ahead of V:
//     during step j the waves read K_{j+1} and V_j while K_{j+3} and V_{j+2}
//     are in flight (three buffers per tensor, d = 64), or K_{j+2} and
//     V_{j+1} (two buffers, d = 128).
//     The buffers are distinct LDS objects and the loop is unrolled by the
//     ring period, so no read names the buffer being filled and the compiler
//     adds no wait on in-flight tiles; with three buffers each step waits only
//     for the copies issued one step earlier, with two for its own.
//   * Within a wave the work is software-pipelined.  Step j runs the softmax
//     of S_j (computed one step earlier) while the matrix cores compute
//     S_{j+1} = K_{j+1} Q^T, then the products P_j V_j, so vector and matrix
//     work of neighbouring tiles overlap.
//   * The reference m of the online softmax is raised only when P formed
//     against it would leave [0, 2^16] in a tile (a tile's row sum is checked
//     as it is formed; the row max is taken only then).  O~, l and L all use
//     the same m, so this is the same algebra as the method's rescale; P is
//     bounded by 2^16 instead of 1, and the per-tile row max and the O~
//     rescale become rare.  (fwd_pipe256_kernel raises m when the row max
//     exceeds it by more than kLazyMax.)
constexpr float kLazyMax = 8.0f;

template <int D, bool CAUSAL, bool SPARSE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(D == 64 && !SPARSE ? 3 : 2, D == 64 && !SPARSE ? 3 : 2)))
void fwd_pipe_kernel(const FwdParams p) {
    constexpr int NW = 4, ROWS = 32 * NW, BC = 64;
    constexpr int KSD = D / 16;          // MFMA reduction steps over the head dim
    constexpr int NBD = D / 32;          // 32-wide blocks of the head dim (O^T)
    constexpr int RB = 2 * D;            // bytes per LDS tile row
    constexpr int kTile = BC * RB;
    constexpr int RPI = 1024 / RB;       // tile rows per wave copy instruction
    constexpr int CPR = RB / 16;         // 16-byte chunks per row
    constexpr int PERW = kTile / 1024 / NW;
    static_assert(PERW >= 1 && kTile % (1024 * NW) == 0, "tile / waves mismatch");
    // K/V ring depth: three tiles per tensor at d = 64 (48 KiB, three
    // workgroups per CU), two at d = 128 (64 KiB, two per CU), whose steps
    // issue their copies at their start and wait for them at their end.
    constexpr int NRING = D == 128 ? 2 : 3;
    constexpr int kTile2 = NRING == 3 ? kTile : 16;
    __shared__ __attribute__((aligned(16))) char Kb0[kTile], Kb1[kTile], Kb2[kTile2];
    __shared__ __attribute__((aligned(16))) char Vb0[kTile], Vb1[kTile], Vb2[kTile2];
    FA2_LDS char* const K0 = (FA2_LDS char*)Kb0;
    FA2_LDS char* const K1 = (FA2_LDS char*)Kb1;
    FA2_LDS char* const K2 = (FA2_LDS char*)Kb2;
    FA2_LDS char* const V0 = (FA2_LDS char*)Vb0;
    FA2_LDS char* const V1 = (FA2_LDS char*)Vb1;
    FA2_LDS char* const V2 = (FA2_LDS char*)Vb2;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int li = lane & 31;

    const int BH = p.B * p.Hq;
    const int level = blockIdx.x / BH;
    const int bh = blockIdx.x - level * BH;
    const int qtile = p.n_qtiles - 1 - level;
    int b, hq;
    level_head(bh, p.Hq, p.G, p.B, b, hq);
    const int hk = hq / p.G;
    const int N = p.N;
    const size_t qhead = ((size_t)b * p.Hq + hq) * (size_t)N * D;
    const size_t khead = ((size_t)b * p.Hkv + hk) * (size_t)N * D;
    const uint16_t* Kh = p.K + khead;
    const uint16_t* Vh = p.V + khead;

    const int q0 = qtile * ROWS;
    const int wq0 = q0 + 32 * wave;
    const int q = wq0 + li;

    el8 qf[KSD];
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
        u32x4 v = {0, 0, 0, 0};
        if (q < N) v = global_load16(p.Q + qhead + (size_t)q * D + 16 * ks + 8 * g);
        qf[ks] = as_el8(v);
    }

    // Tiles the workgroup streams, and tiles this wave computes on.
    //   Dense: tiles 0 .. n_kv-1 (causal: up to the workgroup's last row).
    //   Block-sparse: the workgroup's 128 rows are one mask block; the list
    //   entries 0 .. n_kv-1 are the tiles of every key block its mask row
    //   keeps (causal: the blocks at or below the diagonal).  A wave computes
    //   every entry up to its own causal limit, so the score-ahead pipeline
    //   below stays the dense one.
    int n_kv, n_w;
    FA2_LDS uint16_t* tl = nullptr;
    if constexpr (SPARSE) {
        static_assert(ROWS == kSparseBlock && 2 * BC == kSparseBlock, "one mask block, two tiles per block");
        __shared__ uint16_t tl_arr[kSparseMaxN / BC];
        __shared__ int tl_count;
        tl = (FA2_LDS uint16_t*)tl_arr;
        if (wave == 0) {
            const int r0 = q0 / kSparseBlock, nb = p.nb;
            const int n = build_tile_list(tl, nb, (N + BC - 1) / BC, lane, [&](int c) {
                return p.bmask[(size_t)r0 * nb + c] != 0 && (!CAUSAL || c <= r0) ? 1 : 0;
            });
            if (lane == 0) tl_count = n;
        }
        __syncthreads();
        n_kv = __builtin_amdgcn_readfirstlane(tl_count);
        n_w = wq0 >= N ? 0 : n_kv;
        if (CAUSAL) {
            const int t_last = min(wq0 + 31, N - 1) / BC;
            while (n_w > 0 && (tl[n_w - 1] & 0xfff) > t_last) --n_w;
            n_w = __builtin_amdgcn_readfirstlane(n_w);
        }
    } else {
        n_kv = CAUSAL ? (min(q0 + ROWS, N) - 1) / BC + 1 : (N + BC - 1) / BC;
        n_w = wq0 >= N ? 0 : CAUSAL ? min(wq0 + 31, N - 1) / BC + 1 : n_kv;
    }
    // Key tile of step j.
    auto tile_at = [&](int j) -> int {
        if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)(tl[j] & 0xfff));
        else return j;
    };

    // Copy tile t of K or V into LDS.  Lane i of a copy instruction writes
    // bytes 16*i.. of its 1 KiB (tile row R + i / CPR, 16-byte slot i % CPR),
    // so it fetches the chunk the swizzle puts in that slot.  R is a multiple
    // of RPI, and for these row strides swz(R + r) = swz(r) ^ swz(R) for
    // r < RPI.  Rows past the end repeat row N-1 (their keys are masked).
    // Byte offsets of this lane's chunks in a whole tile (held for the loop);
    // only the tile that ends past N recomputes them, clamped.
    uint32_t off_full[PERW];
#pragma unroll
    for (int i = 0; i < PERW; ++i) {
        const int R = (wave * PERW + i) * RPI;
        const int lr = lane / CPR, lc = 16 * ((lane % CPR) ^ swz<D>(lane / CPR));
        off_full[i] = (uint32_t)((R + lr) * RB + (lc ^ (16 * swz<D>(R))));
    }
    auto copy_tile = [&](const uint16_t* head, int t, FA2_LDS char* dst) {
        const int kv0 = t * BC;
        const char* base = reinterpret_cast<const char*>(head + (size_t)kv0 * D);
        const int last = N - 1 - kv0;
        if (last >= BC - 1) {
#pragma unroll
            for (int i = 0; i < PERW; ++i) copy_to_lds16(base, off_full[i], dst + (wave * PERW + i) * 1024);
        } else {
            int lr = lane / CPR, lc = 16 * ((lane % CPR) ^ swz<D>(lane / CPR));
            asm volatile("" : "+v"(lr), "+v"(lc));
#pragma unroll
            for (int i = 0; i < PERW; ++i) {
                const int R = (wave * PERW + i) * RPI;
                const uint32_t off = (uint32_t)(min(R + lr, last) * RB + (lc ^ (16 * swz<D>(R))));
                copy_to_lds16(base, off, dst + (wave * PERW + i) * 1024);
            }
        }
    };

    // The swizzle only flips bits 4.. of a row's byte offset below RB, so the
    // operand addresses are a per-lane base XOR a constant: 32*ks for K rows
    // (chunk 2*ks + g), 64*db for V columns.  The bases are rebuilt per step
    // (opaque to the compiler) rather than holding one register per address.
    auto scores = [&](const FA2_LDS char* Ks, f32x16 (&s)[2]) {
        int kb = li * RB + 16 * (g ^ swz<D>(li));
        asm volatile("" : "+v"(kb));
        s[0] = zero16();
        s[1] = zero16();
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
            for (int bs = 0; bs < 2; ++bs) {
                const u32x4 a = lds_load16(Ks + 32 * bs * RB + (kb ^ (32 * ks)));
                s[bs] = mfma32(as_el8(a), qf[ks], s[bs]);
            }
    };

    auto mask = [&](int j, f32x16 (&s)[2]) {
        const int kv0 = tile_at(j) * BC;
        if ((kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > wq0)) {
            // Element (bs, r) holds key kv0 + 4g + off with off a constant; it
            // is masked when the key exceeds min(q, N - 1) (causal) or N - 1,
            // i.e. when off > lim: one compare and one select per element.
            const int lim = (CAUSAL ? min(q, N - 1) : N - 1) - kv0 - 4 * g;
#pragma unroll
            for (int bs = 0; bs < 2; ++bs)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[bs][r] = 32 * bs + 8 * (r >> 2) + (r & 3) > lim ? kNegInf : s[bs][r];
        }
    };

    f32x16 o[NBD];
#pragma unroll
    for (int i = 0; i < NBD; ++i) o[i] = zero16();
    float m_run = kNegInf;   // reference max of c * S (log2 domain), equal in lanes l and l ^ 32
    float l_run = 0.f;       // this lane's half of the row sum, relative to m_run

    // P = exp2(c S - m) packed to bf16 (the B operand of the P V product),
    // against the current reference m and summed as it is formed, without a
    // row max in the common case: only when some lane's tile sum leaves
    // [0, 2^16] does the tile's max raise m (and rescale O~ and l), and P is
    // formed again.  So P stays at most 2^16 (no overflow in P, O~ or
    // l), and the first tile, with m = -inf, always takes the max path.  S is
    // left in place for that path.  Returns the rescale factor; lsum gets this
    // lane's half of the tile's row sum.
    auto softmax_nomax = [&](const f32x16 (&s)[2], uint32_t (&pp)[2][8], float& lsum) -> float {
        constexpr float kMaxTileSum = 65536.f;
        auto form = [&](float m_sub) {
            float ls = 0.f;
#pragma unroll
            for (int bs = 0; bs < 2; ++bs)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float t0 = exp2_fast(fmaf(s[bs][r], p.c, -m_sub));
                    const float t1 = exp2_fast(fmaf(s[bs][r + 1], p.c, -m_sub));
                    pp[bs][r >> 1] = pack_el(t0, t1);
                    ls += t0 + t1;
                }
            return ls;
        };
        // With m = -inf a finite reference far below any score sends the tile
        // to the max path (exp2 overflows); masked scores still give 0.
        float ls = form(m_run == kNegInf ? -0x1.0p100f : m_run);
        if (__builtin_amdgcn_ballot_w64(!(ls <= kMaxTileSum)) == 0) {
            lsum = ls;
            return 1.f;
        }
        float mx = kNegInf;
#pragma unroll
        for (int bs = 0; bs < 2; ++bs)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[bs][r]);
        mx = max_halves(mx) * p.c;
        const float m_new = fmaxf(mx, m_run);
        const float alpha = m_new == m_run ? 1.f : exp2_fast(m_run - m_new);
        m_run = m_new;
        lsum = form(m_new == kNegInf ? 0.f : m_new);
        return alpha;
    };


    // O^T += V^T P^T: V^T fragments by transposed reads of the row-major V tile
    // (rows 16*kk + 4*g + j16/4 and +8, columns 32*db + 16*half + 4*(j16 % 4)).
    auto pv = [&](const FA2_LDS char* Vs, const uint32_t (&pp)[2][8]) {
        const int j16 = lane & 15;
        const int x = 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1);    // chunk within a 32-column block
        const int r1 = 4 * g + (j16 >> 2), r2 = r1 + 8;
        int vb1 = r1 * RB + 8 * (j16 & 1) + 16 * (x ^ swz<D>(r1));
        int vb2 = r2 * RB + 8 * (j16 & 1) + 16 * (x ^ swz<D>(r2));
        asm volatile("" : "+v"(vb1), "+v"(vb2));
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int bs = kk >> 1, h = kk & 1;
            const el8 bfrag = as_el8(u32x4{pp[bs][4 * h], pp[bs][4 * h + 1], pp[bs][4 * h + 2], pp[bs][4 * h + 3]});
#pragma unroll
            for (int db = 0; db < NBD; ++db) {
                const s16x4 t1 = lds_load_tr(Vs + 16 * kk * RB + (vb1 ^ (64 * db)));
                const s16x4 t2 = lds_load_tr(Vs + 16 * kk * RB + (vb2 ^ (64 * db)));
                o[db] = mfma32(cat_tr(t1, t2), bfrag, o[db]);
            }
        }
    };

    // A block-sparse workgroup may have no tile at all: it only writes O = 0, L = -inf.
    if (!SPARSE || n_kv > 0) {
    // ---- prologue: K_0, V_0, K_1 (and, three deep, V_1, K_2) in flight; S_0.
    copy_tile(Kh, tile_at(0), K0);
    copy_tile(Vh, tile_at(0), V0);
    if (1 < n_kv) {
        copy_tile(Kh, tile_at(1), K1);
        if (NRING == 3) copy_tile(Vh, tile_at(1), V1);
    }
    if (NRING == 3 && 2 < n_kv) copy_tile(Kh, tile_at(2), K2);
    wait_vm_all();
    __syncthreads();
    f32x16 sa[2], sb[2];       // scores of the current and the next tile, alternating
    scores(K0, sa);
    __syncthreads();          // K_0's buffer is refilled in step 0 (K_3, or K_2 two deep)

    {
    // Step j: softmax of S_j (s_cur) with S_{j+1} = K_{j+1} Q^T (into s_next),
    // then P_j V_j.  Past a wave's last tile the step only copies; S_{j+1} of a
    // tile the wave does not visit is computed from whatever its buffer holds
    // and never used.
    auto step = [&](int j, const FA2_LDS char* Ks, const FA2_LDS char* Vs, FA2_LDS char* Kw, FA2_LDS char* Vw,
                    f32x16 (&s_cur)[2], f32x16 (&s_next)[2]) __attribute__((always_inline)) {
        // Copies past the last tile repeat it into a released buffer that is
        // never read, so every step issues and waits for the same count.
        copy_tile(Kh, tile_at(min(j + NRING, n_kv - 1)), Kw);
        copy_tile(Vh, tile_at(min(j + NRING - 1, n_kv - 1)), Vw);
        if (j < n_w) {
            // Block-sparse: no scores for a list entry past this wave's last
            // (computed one step ahead, in step j - 1).
            const bool own_next = !SPARSE || j + 1 < n_w;
            mask(j, s_cur);
            uint32_t pp[2][8];
            // Raised priority while this wave interleaves S_{j+1} with the
            // softmax of S_j, normal for the P V products: the other wave on the
            // SIMD then fills the matrix unit's idle slots of the mixed phase.
            __builtin_amdgcn_s_setprio(1);
            if (own_next) scores(Ks, s_next);
            {
                float lsum;
                const float alpha = softmax_nomax(s_cur, pp, lsum);
                // Materialize P here, beside the S_{j+1} products, rather than
                // letting the compiler sink the exponentials below the branch.
#pragma unroll
                for (int bs = 0; bs < 2; ++bs)
#pragma unroll
                    for (int r = 0; r < 8; ++r) asm volatile("" ::"v"(pp[bs][r]));
                if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
                    for (int i = 0; i < NBD; ++i)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
                }
                l_run = fmaf(l_run, alpha, lsum);
                __builtin_amdgcn_s_setprio(0);
                pv(Vs, pp);
            }
        }
        if constexpr (NRING == 3) wait_vm_keep<2 * PERW>();   // K_{j+2} and V_{j+1}, issued one step earlier, have landed
        else wait_vm_all();                                 // K_{j+2} and V_{j+1}, issued at this step's start
        barrier_lds();
    };

    if constexpr (NRING == 2) {
        for (int j = 0; j < n_kv; j += 2) {
            step(j, K1, V0, K0, V1, sa, sb);
            if (j + 1 < n_kv) step(j + 1, K0, V1, K1, V0, sb, sa);
        }
    } else
    // Unrolled by six: three buffer phases times two score arrays.  Each step
    // after the first is guarded on its own rather than leaving the loop with
    // a break: with six exits the compiler copied the score arrays into fixed
    // registers at every step instead of alternating them.
    for (int j = 0; j < n_kv; j += 6) {
        step(j, K1, V0, K0, V2, sa, sb);
        if (j + 1 < n_kv) step(j + 1, K2, V1, K1, V0, sb, sa);
        if (j + 2 < n_kv) step(j + 2, K0, V2, K2, V1, sa, sb);
        if (j + 3 < n_kv) step(j + 3, K1, V0, K0, V2, sb, sa);
        if (j + 4 < n_kv) step(j + 4, K2, V1, K1, V0, sa, sb);
        if (j + 5 < n_kv) step(j + 5, K0, V2, K2, V1, sb, sa);
    }
    }
    wait_vm_all();
    }

    // ---- epilogue: O = O~ / l, L = ln2 * (m + log2 l); a block-sparse row
    // without any unmasked key has l = 0: O = 0 and L = -inf.
    if (SPARSE ? wq0 < N : n_w > 0) {
        const float l_tot = sum_halves(l_run);
        const float inv = SPARSE && !(l_tot > 0.f) ? 0.f : 1.0f / l_tot;
        if (q < N) {
            store_o_row<NBD>(p.O + qhead + (size_t)q * D, p.Olo ? p.Olo + qhead + (size_t)q * D : nullptr,
                             o, inv, g);
            if (g == 0)
                p.L[((size_t)b * p.Hq + hq) * N + q] =
                    SPARSE && !(l_tot > 0.f) ? kNegInf : (m_run + log2f(l_tot)) * kLn2;
        }
    }
}

// The pipelined forward at d = 256: the tile pipeline of fwd_pipe_kernel with
// 32-key K/V tiles (16 KiB each, three deep per tensor), one score block per
// step, and 4 waves (one per SIMD, 128 rows per workgroup: the O~ accumulator
// alone takes 128 registers).  With one wave per SIMD nothing else hides a
// wave's latencies, so each step is issued as fixed slot programs (below).
// Block-sparse (SPARSE): a workgroup is exactly one 128-row mask block, so it
// streams the 32-key tiles of the key blocks its mask row keeps (causal: at
// or below the diagonal) from an LDS list and runs the dense step program on
// them; a workgroup whose list is empty writes O = 0 and L = -inf.
template <bool CAUSAL, bool SPARSE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void fwd_pipe256_kernel(const FwdParams p) {
    constexpr int D = 256;
    constexpr int NW = 4, ROWS = 32 * NW, BC = 32;
    constexpr int NBS = BC / 32;         // 32-key score blocks per tile
    constexpr int KSD = D / 16;          // MFMA reduction steps over the head dim
    constexpr int NBD = D / 32;          // 32-wide blocks of the head dim (O^T)
    constexpr int RB = 2 * D;            // bytes per LDS tile row
    constexpr int kTile = BC * RB;
    constexpr int RPI = 1024 / RB;       // tile rows per wave copy instruction
    constexpr int CPR = RB / 16;         // 16-byte chunks per row
    constexpr int PERW = kTile / 1024 / NW;
    static_assert(PERW >= 1 && kTile % (1024 * NW) == 0, "tile / waves mismatch");
    __shared__ __attribute__((aligned(16))) char Kb0[kTile], Kb1[kTile], Kb2[kTile];
    __shared__ __attribute__((aligned(16))) char Vb0[kTile], Vb1[kTile], Vb2[kTile];
    FA2_LDS char* const K0 = (FA2_LDS char*)Kb0;
    FA2_LDS char* const K1 = (FA2_LDS char*)Kb1;
    FA2_LDS char* const K2 = (FA2_LDS char*)Kb2;
    FA2_LDS char* const V0 = (FA2_LDS char*)Vb0;
    FA2_LDS char* const V1 = (FA2_LDS char*)Vb1;
    FA2_LDS char* const V2 = (FA2_LDS char*)Vb2;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int li = lane & 31;

    const int BH = p.B * p.Hq;
    const int level = blockIdx.x / BH;
    const int bh = blockIdx.x - level * BH;
    const int qtile = p.n_qtiles - 1 - level;
    int b, hq;
    level_head(bh, p.Hq, p.G, p.B, b, hq);
    const int hk = hq / p.G;
    const int N = p.N;
    const size_t qhead = ((size_t)b * p.Hq + hq) * (size_t)N * D;
    const size_t khead = ((size_t)b * p.Hkv + hk) * (size_t)N * D;
    const uint16_t* Kh = p.K + khead;
    const uint16_t* Vh = p.V + khead;

    const int q0 = qtile * ROWS;
    const int wq0 = q0 + 32 * wave;
    const int q = wq0 + li;

    el8 qf[KSD];
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
        u32x4 v = {0, 0, 0, 0};
        if (q < N) v = global_load16(p.Q + qhead + (size_t)q * D + 16 * ks + 8 * g);
        qf[ks] = as_el8(v);
    }

    // Tiles the workgroup streams, and tiles this wave computes on (block-
    // sparse: entries of the list, up to this wave's causal limit).
    int n_kv, n_w;
    FA2_LDS uint16_t* tl = nullptr;
    if constexpr (SPARSE) {
        static_assert(ROWS == kSparseBlock && kSparseBlock % BC == 0, "one mask block per workgroup");
        constexpr int TPB = kSparseBlock / BC;
        __shared__ uint16_t tl_arr[kSparseMaxN / BC];
        __shared__ int tl_count;
        tl = (FA2_LDS uint16_t*)tl_arr;
        if (wave == 0) {
            const int r0 = q0 / kSparseBlock, nb = p.nb;
            const int n = build_block_tiles<TPB>(tl, nb, (N + BC - 1) / BC, lane, [&](int c) {
                return p.bmask[(size_t)r0 * nb + c] != 0 && (!CAUSAL || c <= r0);
            });
            if (lane == 0) tl_count = n;
        }
        __syncthreads();
        n_kv = __builtin_amdgcn_readfirstlane(tl_count);
        n_w = wq0 >= N ? 0 : n_kv;
        if (CAUSAL) {
            const int t_last = min(wq0 + 31, N - 1) / BC;
            while (n_w > 0 && (int)tl[n_w - 1] > t_last) --n_w;
            n_w = __builtin_amdgcn_readfirstlane(n_w);
        }
    } else {
        n_kv = CAUSAL ? (min(q0 + ROWS, N) - 1) / BC + 1 : (N + BC - 1) / BC;
        n_w = wq0 >= N ? 0 : CAUSAL ? min(wq0 + 31, N - 1) / BC + 1 : n_kv;
    }
    // Key tile of step j.
    auto tile_at = [&](int j) -> int {
        if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)tl[j]);
        else return j;
    };

    // Copy tile t of K or V into LDS.  Lane i of a copy instruction writes
    // bytes 16*i.. of its 1 KiB (tile row R + i / CPR, 16-byte slot i % CPR),
    // so it fetches the chunk the swizzle puts in that slot.  R is a multiple
    // of RPI, and for these row strides swz(R + r) = swz(r) ^ swz(R) for
    // r < RPI.  Rows past the end repeat row N-1 (their keys are masked).
    // Byte offsets of this lane's chunks in a whole tile (held for the loop);
    // only the tile that ends past N recomputes them, clamped.
    uint32_t off_full[PERW];
#pragma unroll
    for (int i = 0; i < PERW; ++i) {
        const int R = (wave * PERW + i) * RPI;
        const int lr = lane / CPR, lc = 16 * ((lane % CPR) ^ swz<D>(lane / CPR));
        off_full[i] = (uint32_t)((R + lr) * RB + (lc ^ (16 * swz<D>(R))));
    }
    auto copy_tile = [&](const uint16_t* head, int t, FA2_LDS char* dst) {
        const int kv0 = t * BC;
        const char* base = reinterpret_cast<const char*>(head + (size_t)kv0 * D);
        const int last = N - 1 - kv0;
        if (last >= BC - 1) {
#pragma unroll
            for (int i = 0; i < PERW; ++i) copy_to_lds16(base, off_full[i], dst + (wave * PERW + i) * 1024);
        } else {
            int lr = lane / CPR, lc = 16 * ((lane % CPR) ^ swz<D>(lane / CPR));
            asm volatile("" : "+v"(lr), "+v"(lc));
#pragma unroll
            for (int i = 0; i < PERW; ++i) {
                const int R = (wave * PERW + i) * RPI;
                const uint32_t off = (uint32_t)(min(R + lr, last) * RB + (lc ^ (16 * swz<D>(R))));
                copy_to_lds16(base, off, dst + (wave * PERW + i) * 1024);
            }
        }
    };

    // The swizzle only flips bits 4.. of a row's byte offset below RB, so the
    // operand addresses are a per-lane base XOR a constant: 32*ks for K rows
    // (chunk 2*ks + g), 64*db for V columns.  The bases are rebuilt per step
    // (opaque to the compiler) rather than holding one register per address.
    auto scores = [&](const FA2_LDS char* Ks, f32x16 (&s)[NBS]) {
        int kb = li * RB + 16 * (g ^ swz<D>(li));
        asm volatile("" : "+v"(kb));
#pragma unroll
        for (int bs = 0; bs < NBS; ++bs) s[bs] = zero16();
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
            for (int bs = 0; bs < NBS; ++bs) {
                const u32x4 a = lds_load16(Ks + 32 * bs * RB + (kb ^ (32 * ks)));
                s[bs] = mfma32(as_el8(a), qf[ks], s[bs]);
            }
    };

    auto mask = [&](int j, f32x16 (&s)[NBS]) {
        const int kv0 = tile_at(j) * BC;
        if ((kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > wq0)) {
            // As in fwd_pipe_kernel: masked when the constant key offset exceeds lim.
            const int lim = (CAUSAL ? min(q, N - 1) : N - 1) - kv0 - 4 * g;
#pragma unroll
            for (int bs = 0; bs < NBS; ++bs)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[bs][r] = 32 * bs + 8 * (r >> 2) + (r & 3) > lim ? kNegInf : s[bs][r];
        }
    };

    f32x16 o[NBD];
#pragma unroll
    for (int i = 0; i < NBD; ++i) o[i] = zero16();
    float m_run = kNegInf;   // reference max of c * S (log2 domain), equal in lanes l and l ^ 32
    float l_run = 0.f;       // this lane's half of the row sum, relative to m_run

    // A block-sparse workgroup may have no tile at all: it only writes O = 0, L = -inf.
    if (!SPARSE || n_kv > 0) {
    // ---- prologue: K_0, V_0, K_1, V_1, K_2 in flight; S_0.
    copy_tile(Kh, tile_at(0), K0);
    copy_tile(Vh, tile_at(0), V0);
    if (1 < n_kv) {
        copy_tile(Kh, tile_at(1), K1);
        copy_tile(Vh, tile_at(1), V1);
    }
    if (2 < n_kv) copy_tile(Kh, tile_at(2), K2);
    wait_vm_all();
    __syncthreads();
    f32x16 sa[NBS], sb[NBS];       // scores of the current and the next tile, alternating
    scores(K0, sa);
    __syncthreads();          // K_0 is overwritten by K_3 in step 0

    // A step as two fixed slot programs, one matrix product per slot (with
    // one wave per SIMD the issue order is the overlap).  Phase 1 issues the
    // 16 products of S_{j+1}, each K operand read kPf slots ahead, and spreads
    // the softmax of S_j over the slots: the row max in slots 0-3, the new
    // reference max in slot 4, two exponentials and one packing per slot in
    // slots 5-12, and the first V^T reads of phase 2 in slots 12-15.  Phase 2
    // issues the 16 P V products with their operands read kPf slots ahead and
    // one row-sum addition per slot.  A scheduling fence between slots keeps
    // this order; an empty asm that redefines each staged value keeps the
    // compiler from sinking it to its first use.
    constexpr int kPf = 4;
    static_assert(NBS == 1 && KSD == 16 && 2 * NBD == 16, "slot programs for d = 256, 32-key tiles");
    auto pin = [](float& x) { asm volatile("" : "+v"(x)); };
    int pvb1 = 0, pvb2 = 0;
    auto v_bases = [&]() {
        const int j16 = lane & 15;
        const int x = 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1);    // chunk within a 32-column block
        const int r1 = 4 * g + (j16 >> 2), r2 = r1 + 8;
        pvb1 = r1 * RB + 8 * (j16 & 1) + 16 * (x ^ swz<D>(r1));
        pvb2 = r2 * RB + 8 * (j16 & 1) + 16 * (x ^ swz<D>(r2));
        asm volatile("" : "+v"(pvb1), "+v"(pvb2));
    };
    // V^T fragment of P V product k (keys 16 (k / 8) .., head-dim block k % 8).
    auto load_vt = [&](const FA2_LDS char* Vs, int k, s16x4 (&t)[2]) {
        const int kk = k / NBD, db = k % NBD;
        t[0] = lds_load_tr(Vs + 16 * kk * RB + (pvb1 ^ (64 * db)));
        t[1] = lds_load_tr(Vs + 16 * kk * RB + (pvb2 ^ (64 * db)));
    };
    auto phase1 = [&](const FA2_LDS char* Ks, const FA2_LDS char* Vs, f32x16& sc, f32x16& sn, uint32_t (&pp)[8],
                      s16x4 (&vt)[kPf][2]) -> float {
        int kb = li * RB + 16 * (g ^ swz<D>(li));
        asm volatile("" : "+v"(kb));
        v_bases();
        u32x4 ka[kPf];
#pragma unroll
        for (int k = 0; k < kPf; ++k) ka[k] = lds_load16(Ks + (kb ^ (32 * k)));
        sn = zero16();
        float m0 = kNegInf, m1 = kNegInf, m_sub = 0.f, alpha = 1.f;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            const u32x4 a = ka[ks % kPf];
            if (ks + kPf < KSD) ka[ks % kPf] = lds_load16(Ks + (kb ^ (32 * (ks + kPf))));
            sn = mfma32(as_el8(a), qf[ks], sn);
            if (ks < 4) {
                m0 = fmaxf(fmaxf(m0, sc[4 * ks]), sc[4 * ks + 1]);
                m1 = fmaxf(fmaxf(m1, sc[4 * ks + 2]), sc[4 * ks + 3]);
                pin(m0);
                pin(m1);
            } else if (ks == 4) {
                const float mx = max_halves(fmaxf(m0, m1)) * p.c;
                const float m_new = mx > m_run + kLazyMax ? mx : m_run;
                alpha = m_new == m_run ? 1.f : exp2_fast(m_run - m_new);
                m_run = m_new;
                // Block-sparse rows may not have met an unmasked key yet (m = -inf):
                // exp2(-inf - 0) = 0 then, where -inf - (-inf) would be NaN.
                m_sub = SPARSE && m_new == kNegInf ? 0.f : m_new;
                pin(m_sub);
                pin(alpha);
            } else if (ks < 13) {
                const int r = 2 * (ks - 5);
                float e0 = exp2_fast(fmaf(sc[r], p.c, -m_sub));
                float e1 = exp2_fast(fmaf(sc[r + 1], p.c, -m_sub));
                pin(e0);
                pin(e1);
                uint32_t w = pack_el(e0, e1);
                asm volatile("" : "+v"(w));
                pp[r >> 1] = w;
                sc[r] = e0;
                sc[r + 1] = e1;
            }
            if (ks >= KSD - kPf) load_vt(Vs, ks - (KSD - kPf), vt[ks - (KSD - kPf)]);
        }
        __builtin_amdgcn_sched_barrier(0);
        return alpha;
    };
    auto phase2 = [&](const FA2_LDS char* Vs, const uint32_t (&pp)[8], const f32x16& pr, s16x4 (&vt)[kPf][2],
                      float alpha) {
        float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
        for (int k = 0; k < 2 * NBD; ++k) {
            __builtin_amdgcn_sched_barrier(0);
            const int kk = k / NBD, db = k % NBD;
            const s16x4 t1 = vt[k % kPf][0], t2 = vt[k % kPf][1];
            if (k + kPf < 2 * NBD) load_vt(Vs, k + kPf, vt[k % kPf]);
            const el8 bfrag = as_el8(u32x4{pp[4 * kk], pp[4 * kk + 1], pp[4 * kk + 2], pp[4 * kk + 3]});
            o[db] = mfma32(cat_tr(t1, t2), bfrag, o[db]);
            if (k & 1) ls1 += pr[k];
            else ls0 += pr[k];
        }
        __builtin_amdgcn_sched_barrier(0);
        l_run = fmaf(l_run, alpha, ls0 + ls1);
    };

    // Step j: softmax of S_j (s_cur) with S_{j+1} = K_{j+1} Q^T (into s_next),
    // then P_j V_j.  Past a wave's last tile the step only copies; S_{j+1} of a
    // tile the wave does not visit is computed from whatever its buffer holds
    // and never used.
    auto step = [&](int j, const FA2_LDS char* Ks, const FA2_LDS char* Vs, FA2_LDS char* Kw, FA2_LDS char* Vw,
                    f32x16 (&s_cur)[NBS], f32x16 (&s_next)[NBS]) __attribute__((always_inline)) {
        // Copies past the last tile repeat it into a released buffer that is
        // never read, so every step issues and waits for the same count.
        copy_tile(Kh, tile_at(min(j + 3, n_kv - 1)), Kw);
        copy_tile(Vh, tile_at(min(j + 2, n_kv - 1)), Vw);
        if (j < n_w) {
            mask(j, s_cur);
            uint32_t pp[8];
            s16x4 vt[kPf][2];
            const float alpha = phase1(Ks, Vs, s_cur[0], s_next[0], pp, vt);
            if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
                for (int i = 0; i < NBD; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
            }
            phase2(Vs, pp, s_cur[0], vt, alpha);
        }
        wait_vm_keep<2 * PERW>();   // K_{j+2} and V_{j+1}, issued one step earlier, have landed
        barrier_lds();
    };

    // Unrolled by six: three buffer phases times two score arrays.  Each step
    // after the first is guarded on its own rather than leaving the loop with
    // a break: with six exits the compiler copied the score arrays into fixed
    // registers at every step instead of alternating them.
    for (int j = 0; j < n_kv; j += 6) {
        step(j, K1, V0, K0, V2, sa, sb);
        if (j + 1 < n_kv) step(j + 1, K2, V1, K1, V0, sb, sa);
        if (j + 2 < n_kv) step(j + 2, K0, V2, K2, V1, sa, sb);
        if (j + 3 < n_kv) step(j + 3, K1, V0, K0, V2, sb, sa);
        if (j + 4 < n_kv) step(j + 4, K2, V1, K1, V0, sa, sb);
        if (j + 5 < n_kv) step(j + 5, K0, V2, K2, V1, sb, sa);
    }
    wait_vm_all();
    }

    // ---- epilogue: O = O~ / l, L = ln2 * (m + log2 l); a block-sparse row
    // without any unmasked key has l = 0: O = 0 and L = -inf.
    if (SPARSE ? wq0 < N : n_w > 0) {
        const float l_tot = sum_halves(l_run);
        const float inv = SPARSE && !(l_tot > 0.f) ? 0.f : 1.0f / l_tot;
        if (q < N) {
            store_o_row<NBD>(p.O + qhead + (size_t)q * D, p.Olo ? p.Olo + qhead + (size_t)q * D : nullptr,
                             o, inv, g);
            if (g == 0)
                p.L[((size_t)b * p.Hq + hq) * N + q] =
                    SPARSE && !(l_tot > 0.f) ? kNegInf : (m_run + log2f(l_tot)) * kLn2;
        }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
    FwdParams arg = p;
    void* args[] = {&arg};
    if constexpr (D <= 128) {
        // 128-row workgroups of 4 waves: three per CU at d = 64, two at d = 128.
        const int rows = 128;
        arg.n_qtiles = (p.N + rows - 1) / rows;
        const long grid = (long)p.B * p.Hq * arg.n_qtiles;
        const void* fn;
        if (p.bmask) fn = reinterpret_cast<const void*>(&fwd_pipe_kernel<D, CAUSAL, true>);
        else fn = reinterpret_cast<const void*>(&fwd_pipe_kernel<D, CAUSAL, false>);
        return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(2 * rows), args, 0, stream);
    } else {
        arg.n_qtiles = (p.N + 127) / 128;
        const long grid = (long)p.B * p.Hq * arg.n_qtiles;
        const void* fn = p.bmask ? reinterpret_cast<const void*>(&fwd_pipe256_kernel<CAUSAL, true>)
                                 : reinterpret_cast<const void*>(&fwd_pipe256_kernel<CAUSAL, false>);
        return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, stream);
    }
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int d, bool causal, hipStream_t stream) {
    switch (d) {
        case 64: return causal ? launch_fwd_t<64, true>(p, stream) : launch_fwd_t<64, false>(p, stream);
        case 128: return causal ? launch_fwd_t<128, true>(p, stream) : launch_fwd_t<128, false>(p, stream);
        case 256: return causal ? launch_fwd_t<256, true>(p, stream) : launch_fwd_t<256, false>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace FA2_NS
