// fa2_api.hip -- the C ABI of libfa2.so (declared in include/fa2.h).
//
// Argument checking is pure host code that makes no HIP call, so it is
// testable without a GPU (fa2_validate_fwd / fa2_validate_bwd).  The entry
// points check, then fill the kernel parameter blocks and launch on the
// caller's stream.  The library allocates nothing: the backward pass's
// fp32 scratch (D and the dQ accumulator) comes from the caller's workspace.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "fa2.h"
#include "fa2_kernels.h"

// Scratch of fa2_bwd_noalloc: the backward's per-row arrays (-D and L * log2(e))
// for callers that cannot allocate.  Each device holds its own copy for the
// life of the process.  In host code `scratch` names a host-side stand-in, not
// device memory: its device address is looked up per device with
// hipGetSymbolAddress and only that address is passed to kernels.
static constexpr size_t kScratchBytes = FA2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local char g_last_error[256] = "";

fa2_status fail(fa2_status s, const char* fmt, const char* detail = nullptr) {
    if (detail)
        std::snprintf(g_last_error, sizeof g_last_error, fmt, detail);
    else
        std::snprintf(g_last_error, sizeof g_last_error, "%s", fmt);
    return s;
}

constexpr size_t kWorkspaceAlign = 256;
constexpr int kMaxN = 1 << 30;             // keeps every in-kernel row index in int range
constexpr uint64_t kMaxGridThreads = 0xFFFFFFFFull;  // work-items per grid dimension

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool mul_overflows(uint64_t a, uint64_t b, uint64_t* out) {
    if (a != 0 && b > UINT64_MAX / a) return true;
    *out = a * b;
    return false;
}

// Element count of [a, b, c, d]; false on 64-bit overflow.
bool count4(int a, int b, int c, int d, uint64_t* out) {
    uint64_t x;
    if (mul_overflows((uint64_t)a, (uint64_t)b, &x)) return false;
    if (mul_overflows(x, (uint64_t)c, &x)) return false;
    if (mul_overflows(x, (uint64_t)d, &x)) return false;
    *out = x;
    return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, uint64_t abytes, const void* b, uint64_t bbytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bbytes && y < x + abytes;
}

struct Sizes {
    uint64_t q_elems = 0, kv_elems = 0, rows = 0;  // rows = B * Hq * N
    uint64_t rows_pad = 0;                          // B * Hq * N rounded up per head
};

// Rows of the per-row workspace arrays of one head: N rounded up to a
// multiple of kBwdRowPad.
int padded_rows(int N) { return (N + fa2::kBwdRowPad - 1) / fa2::kBwdRowPad * fa2::kBwdRowPad; }

// Shared checks of sizes, head dim, scale and grid limits.  Returns FA2_OK
// with *empty set when there is nothing to compute.
fa2_status check_problem(int B, int Hq, int Hkv, int N, int d, float scale, bool* empty,
                         Sizes* sz) {
    *empty = false;
    if (B < 0 || Hq < 0 || Hkv < 0 || N < 0 || d < 0)
        return fail(FA2_ERR_INVALID_ARGUMENT, "negative size");
    if (B == 0 || Hq == 0 || N == 0) {
        *empty = true;
        return FA2_OK;
    }
    if (Hkv < 1) return fail(FA2_ERR_INVALID_ARGUMENT, "Hkv must be >= 1");
    if (Hq % Hkv != 0) return fail(FA2_ERR_INVALID_ARGUMENT, "Hq must be a multiple of Hkv");
    if (d != 64 && d != 128 && d != 256)
        return fail(FA2_ERR_UNSUPPORTED, "head dim must be 64, 128 or 256");
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(FA2_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
    if (!count4(B, Hq, N, d, &sz->q_elems) || !count4(B, Hkv, N, d, &sz->kv_elems) ||
        !count4(B, Hq, N, 1, &sz->rows) || sz->q_elems > (UINT64_MAX >> 3))
        return fail(FA2_ERR_INVALID_ARGUMENT, "element count overflows 64 bits");
    if (N > kMaxN) return fail(FA2_ERR_UNSUPPORTED, "N above 2^30");
    if (!count4(B, Hq, padded_rows(N), 1, &sz->rows_pad) || sz->rows_pad > (UINT64_MAX >> 4))
        return fail(FA2_ERR_INVALID_ARGUMENT, "element count overflows 64 bits");
    // Largest grid launched: forward B*Hq*ceil(N/128) or backward B*Hkv*ceil(N/64), 256 threads.
    const uint64_t tiles = (uint64_t)B * (uint64_t)Hq * (uint64_t)((N + 63) / 64);
    if (tiles * 256u > kMaxGridThreads) return fail(FA2_ERR_UNSUPPORTED, "grid too large");
    return FA2_OK;
}

fa2_status validate_fwd(const void* Q, const void* K, const void* V, const void* O, const float* L,
                        int B, int Hq, int Hkv, int N, int d, float scale, bool* empty, Sizes* sz) {
    fa2_status s = check_problem(B, Hq, Hkv, N, d, scale, empty, sz);
    if (s != FA2_OK || *empty) return s;
    const void* ptrs[5] = {Q, K, V, O, L};
    const char* names[5] = {"Q", "K", "V", "O", "L"};
    for (int i = 0; i < 5; ++i) {
        if (!ptrs[i]) return fail(FA2_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
        if (!aligned16(ptrs[i])) return fail(FA2_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", names[i]);
    }
    const uint64_t qb = sz->q_elems * 2, kb = sz->kv_elems * 2, lb = sz->rows * 4;
    if (overlaps(O, qb, Q, qb) || overlaps(O, qb, K, kb) || overlaps(O, qb, V, kb))
        return fail(FA2_ERR_INVALID_ARGUMENT, "O aliases an input");
    if (overlaps(L, lb, Q, qb) || overlaps(L, lb, K, kb) || overlaps(L, lb, V, kb))
        return fail(FA2_ERR_INVALID_ARGUMENT, "L aliases an input");
    if (overlaps(O, qb, L, lb)) return fail(FA2_ERR_INVALID_ARGUMENT, "O aliases L");
    return FA2_OK;
}

struct WorkspaceLayout {
    size_t d_off, l2_off, dq_off, total;
};

// D [B*Hq*Npad] fp32, then L * log2(e) [B*Hq*Npad] fp32, each on a 256-byte
// boundary; in the atomic-dQ mode also the dQ accumulator [B*Hq*N*d] fp32.
WorkspaceLayout workspace_layout(uint64_t rows_pad, uint64_t q_elems, bool atomic) {
    WorkspaceLayout w;
    w.d_off = 0;
    w.l2_off = align_up(rows_pad * 4, kWorkspaceAlign);
    w.dq_off = w.l2_off + align_up(rows_pad * 4, kWorkspaceAlign);
    w.total = w.dq_off + (atomic ? align_up(q_elems * 4, kWorkspaceAlign) : 0);
    return w;
}

fa2_status validate_bwd(const void* Q, const void* K, const void* V, const void* O, const float* L,
                        const void* dO, const void* dQ, const void* dK, const void* dV,
                        const void* ws, size_t ws_bytes, int B, int Hq, int Hkv, int N, int d,
                        float scale, bool atomic, bool* empty, Sizes* sz,
                        bool static_ws = false) {
    fa2_status s = check_problem(B, Hq, Hkv, N, d, scale, empty, sz);
    if (s != FA2_OK || *empty) return s;
    const void* ptrs[9] = {Q, K, V, O, L, dO, dQ, dK, dV};
    const char* names[9] = {"Q", "K", "V", "O", "L", "dO", "dQ", "dK", "dV"};
    for (int i = 0; i < 9; ++i) {
        if (!ptrs[i]) return fail(FA2_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
        if (!aligned16(ptrs[i])) return fail(FA2_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", names[i]);
    }
    const WorkspaceLayout wl = workspace_layout(sz->rows_pad, sz->q_elems, atomic);
    // static_ws: the library's own scratch array, checked by the caller of this
    // function against its fixed size; only the caller's buffers are checked here.
    if (!static_ws) {
        if (!ws) return fail(FA2_ERR_INVALID_ARGUMENT, "workspace is NULL");
        if ((reinterpret_cast<uintptr_t>(ws) & (kWorkspaceAlign - 1)) != 0)
            return fail(FA2_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
        if (ws_bytes < wl.total) return fail(FA2_ERR_INVALID_ARGUMENT, "workspace too small");
    }
    const uint64_t qb = sz->q_elems * 2, kb = sz->kv_elems * 2, lb = sz->rows * 4;
    const void* ins[6] = {Q, K, V, O, L, dO};
    const uint64_t in_bytes[6] = {qb, kb, kb, qb, lb, qb};
    const void* outs[4] = {dQ, dK, dV, ws};
    const uint64_t out_bytes[4] = {qb, kb, kb, static_ws ? 0 : wl.total};
    const char* out_names[4] = {"dQ", "dK", "dV", "workspace"};
    for (int o = 0; o < (static_ws ? 3 : 4); ++o) {
        for (int i = 0; i < 6; ++i)
            if (overlaps(outs[o], out_bytes[o], ins[i], in_bytes[i]))
                return fail(FA2_ERR_INVALID_ARGUMENT, "%s aliases an input", out_names[o]);
        for (int o2 = o + 1; o2 < (static_ws ? 3 : 4); ++o2)
            if (overlaps(outs[o], out_bytes[o], outs[o2], out_bytes[o2]))
                return fail(FA2_ERR_INVALID_ARGUMENT, "%s aliases another output", out_names[o]);
    }
    return FA2_OK;
}

// O_lo of the split-O entry points: present, 16-byte aligned, and (in the
// forward, where it is an output) not overlapping the inputs.  The forward
// also checks it against O and L, the backward against its outputs.
fa2_status validate_olo(const void* Olo, const void* Q, const void* K, const void* V, const Sizes& sz) {
    if (!Olo) return fail(FA2_ERR_INVALID_ARGUMENT, "O_lo is NULL");
    if (!aligned16(Olo)) return fail(FA2_ERR_INVALID_ARGUMENT, "O_lo is not 16-byte aligned");
    const uint64_t qb = sz.q_elems * 2, kb = sz.kv_elems * 2;
    if (overlaps(Olo, qb, Q, qb) || overlaps(Olo, qb, K, kb) || overlaps(Olo, qb, V, kb))
        return fail(FA2_ERR_INVALID_ARGUMENT, "O_lo aliases Q, K or V");
    return FA2_OK;
}

// Block-sparse attention: the block mask [nb, nb] bytes, nb = ceil(N / 128).
// It must be present, N at most kSparseMaxN (the kernels hold one mask row or
// column of tiles in LDS), and no output may overlap it.
fa2_status validate_mask(const unsigned char* bmask, int N, const void* const* outs,
                         const uint64_t* out_bytes, int n_outs) {
    if (!bmask) return fail(FA2_ERR_INVALID_ARGUMENT, "block_mask is NULL");
    if (N > fa2::kSparseMaxN) return fail(FA2_ERR_UNSUPPORTED, "block-sparse attention needs N <= 262144");
    const uint64_t nb = (uint64_t)((N + fa2::kSparseBlock - 1) / fa2::kSparseBlock);
    for (int o = 0; o < n_outs; ++o)
        if (overlaps(outs[o], out_bytes[o], bmask, nb * nb))
            return fail(FA2_ERR_INVALID_ARGUMENT, "an output aliases block_mask");
    return FA2_OK;
}

constexpr double kLog2e = 1.4426950408889634074;

// Device address of `scratch` on each device, looked up on the first
// fa2_bwd_noalloc call made with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

fa2_status scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FA2_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(FA2_ERR_UNSUPPORTED, "device index above 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(FA2_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FA2_OK;
}

}  // namespace

extern "C" {

const char* fa2_status_string(int status) {
    switch (status) {
        case FA2_OK: return "FA2_OK";
        case FA2_ERR_INVALID_ARGUMENT: return "FA2_ERR_INVALID_ARGUMENT";
        case FA2_ERR_UNSUPPORTED: return "FA2_ERR_UNSUPPORTED";
        case FA2_ERR_HIP: return "FA2_ERR_HIP";
    }
    return "unknown status";
}

const char* fa2_last_error(void) { return g_last_error; }

fa2_status fa2_validate_fwd(const void* Q, const void* K, const void* V, const void* O,
                            const float* L, int B, int Hq, int Hkv, int N, int d, int causal,
                            float scale) {
    (void)causal;
    g_last_error[0] = '\0';
    bool empty;
    Sizes sz;
    return validate_fwd(Q, K, V, O, L, B, Hq, Hkv, N, d, scale, &empty, &sz);
}

fa2_status fa2_validate_bwd(const void* Q, const void* K, const void* V, const void* O,
                            const float* L, const void* dO, const void* dQ, const void* dK,
                            const void* dV, const void* workspace, size_t workspace_bytes, int B,
                            int Hq, int Hkv, int N, int d, int causal, float scale) {
    (void)causal;
    g_last_error[0] = '\0';
    bool empty;
    Sizes sz;
    return validate_bwd(Q, K, V, O, L, dO, dQ, dK, dV, workspace, workspace_bytes, B, Hq, Hkv, N,
                        d, scale, false, &empty, &sz);
}

size_t fa2_bwd_stages_workspace_bytes(unsigned stages, int B, int Hq, int Hkv, int N, int d) {
    if ((stages & FA2_BWD_ALL) == 0 || (stages & ~(FA2_BWD_ALL | FA2_BWD_DQ_ATOMIC)) != 0) return 0;
    if (B < 0 || Hq < 0 || Hkv < 0 || N < 0 || d < 0) return 0;
    if (B == 0 || Hq == 0 || N == 0) return 0;
    if (Hkv < 1 || Hq % Hkv != 0) return 0;
    uint64_t q_elems, rows_pad;
    if (N > kMaxN || !count4(B, Hq, N, d, &q_elems) || !count4(B, Hq, padded_rows(N), 1, &rows_pad) ||
        q_elems > (UINT64_MAX >> 3) || rows_pad > (UINT64_MAX >> 4))
        return 0;
    return workspace_layout(rows_pad, q_elems, (stages & FA2_BWD_DQ_ATOMIC) != 0).total;
}

size_t fa2_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
    return fa2_bwd_stages_workspace_bytes(FA2_BWD_ALL, B, Hq, Hkv, N, d);
}

}  // extern "C"

namespace {

// The forward for either element format (f16: the kernels compiled into fa2_f16).
// bmask: NULL for dense attention; `sparse` says whether the caller is a
// block-sparse entry point (which then requires a mask).
fa2_status fwd_impl(bool f16, bool sparse, const unsigned char* bmask, const void* Q, const void* K,
                    const void* V, void* O, float* L, int B, int Hq, int Hkv, int N, int d,
                    int causal, float scale, void* stream, bool with_olo = false, void* Olo = nullptr) {
    g_last_error[0] = '\0';
    bool empty;
    Sizes sz;
    fa2_status s = validate_fwd(Q, K, V, O, L, B, Hq, Hkv, N, d, scale, &empty, &sz);
    if (s != FA2_OK || empty) return s;
    if (with_olo) {
        s = validate_olo(Olo, Q, K, V, sz);
        if (s != FA2_OK) return s;
        if (overlaps(Olo, sz.q_elems * 2, O, sz.q_elems * 2) || overlaps(Olo, sz.q_elems * 2, L, sz.rows * 4))
            return fail(FA2_ERR_INVALID_ARGUMENT, "O_lo aliases another output");
    }
    if (sparse) {
        const void* outs[2] = {O, L};
        const uint64_t ob[2] = {sz.q_elems * 2, sz.rows * 4};
        s = validate_mask(bmask, N, outs, ob, 2);
        if (s != FA2_OK) return s;
    }
    fa2::FwdParams p;
    p.Q = static_cast<const uint16_t*>(Q);
    p.K = static_cast<const uint16_t*>(K);
    p.V = static_cast<const uint16_t*>(V);
    p.O = static_cast<uint16_t*>(O);
    p.Olo = static_cast<uint16_t*>(Olo);
    p.L = L;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.N = N;
    p.G = Hq / Hkv;
    p.n_qtiles = 0;     // set by the launcher for its workgroup shape
    p.c = (float)((double)scale * kLog2e);
    p.bmask = sparse ? bmask : nullptr;
    p.nb = (N + fa2::kSparseBlock - 1) / fa2::kSparseBlock;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = f16 ? fa2_f16::launch_fwd(p, d, causal != 0, st) : fa2::launch_fwd(p, d, causal != 0, st);
    if (e != hipSuccess) return fail(FA2_ERR_HIP, "%s", hipGetErrorString(e));
    return FA2_OK;
}

// The backward stages for either element format.
fa2_status bwd_impl(bool f16, unsigned stages, bool sparse, const unsigned char* bmask,
                    const void* Q, const void* K, const void* V, const void* O, const float* L,
                    const void* dO, void* dQ, void* dK, void* dV, void* workspace,
                    size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, int causal,
                    float scale, void* stream, bool with_olo = false, const void* Olo = nullptr) {
    g_last_error[0] = '\0';
    if ((stages & FA2_BWD_ALL) == 0 || (stages & ~(FA2_BWD_ALL | FA2_BWD_DQ_ATOMIC)) != 0)
        return fail(FA2_ERR_INVALID_ARGUMENT,
                    "stage mask must hold at least one stage of FA2_BWD_ALL and no unknown bits");
    bool empty;
    Sizes sz;
    const bool atomic = (stages & FA2_BWD_DQ_ATOMIC) != 0;
    fa2_status s = validate_bwd(Q, K, V, O, L, dO, dQ, dK, dV, workspace, workspace_bytes, B, Hq,
                                Hkv, N, d, scale, atomic, &empty, &sz);
    if (s != FA2_OK || empty) return s;
    const WorkspaceLayout wl = workspace_layout(sz.rows_pad, sz.q_elems, atomic);
    if (with_olo) {
        s = validate_olo(Olo, Q, K, V, sz);
        if (s != FA2_OK) return s;
        const void* outs[4] = {dQ, dK, dV, workspace};
        const uint64_t ob[4] = {sz.q_elems * 2, sz.kv_elems * 2, sz.kv_elems * 2, wl.total};
        for (int o = 0; o < 4; ++o)
            if (overlaps(outs[o], ob[o], Olo, sz.q_elems * 2))
                return fail(FA2_ERR_INVALID_ARGUMENT, "an output aliases O_lo");
    }
    if (sparse) {
        const void* outs[4] = {dQ, dK, dV, workspace};
        const uint64_t ob[4] = {sz.q_elems * 2, sz.kv_elems * 2, sz.kv_elems * 2, wl.total};
        s = validate_mask(bmask, N, outs, ob, 4);
        if (s != FA2_OK) return s;
    }
    fa2::BwdParams p;
    p.Q = static_cast<const uint16_t*>(Q);
    p.K = static_cast<const uint16_t*>(K);
    p.V = static_cast<const uint16_t*>(V);
    p.O = static_cast<const uint16_t*>(O);
    p.Olo = static_cast<const uint16_t*>(Olo);
    p.L = L;
    p.dO = static_cast<const uint16_t*>(dO);
    p.dQ = static_cast<uint16_t*>(dQ);
    p.dK = static_cast<uint16_t*>(dK);
    p.dV = static_cast<uint16_t*>(dV);
    p.Dneg = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.d_off);
    p.L2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.l2_off);
    p.dQacc = atomic ? reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.dq_off) : nullptr;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.N = N;
    p.Npad = padded_rows(N);
    p.G = Hq / Hkv;
    p.scale = scale;
    p.c = (float)((double)scale * kLog2e);
    p.bmask = sparse ? bmask : nullptr;
    p.nb = (N + fa2::kSparseBlock - 1) / fa2::kSparseBlock;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = f16 ? fa2_f16::launch_bwd(p, d, causal != 0, stages, st)
                       : fa2::launch_bwd(p, d, causal != 0, stages, st);
    if (e != hipSuccess) return fail(FA2_ERR_HIP, "%s", hipGetErrorString(e));
    return FA2_OK;
}

}  // namespace

extern "C" {

fa2_status fa2_fwd(const void* Q, const void* K, const void* V, void* O, float* L, int B, int Hq,
                   int Hkv, int N, int d, int causal, float scale, void* stream) {
    return fwd_impl(false, false, nullptr, Q, K, V, O, L, B, Hq, Hkv, N, d, causal, scale, stream);
}

fa2_status fa2_fwd_f16(const void* Q, const void* K, const void* V, void* O, float* L, int B,
                       int Hq, int Hkv, int N, int d, int causal, float scale, void* stream) {
    return fwd_impl(true, false, nullptr, Q, K, V, O, L, B, Hq, Hkv, N, d, causal, scale, stream);
}

fa2_status fa2_bwd(const void* Q, const void* K, const void* V, const void* O, const float* L,
                   const void* dO, void* dQ, void* dK, void* dV, void* workspace,
                   size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, int causal,
                   float scale, void* stream) {
    return bwd_impl(false, FA2_BWD_ALL, false, nullptr, Q, K, V, O, L, dO, dQ, dK, dV, workspace, workspace_bytes,
                    B, Hq, Hkv, N, d, causal, scale, stream);
}

fa2_status fa2_bwd_stages(unsigned stages, const void* Q, const void* K, const void* V,
                          const void* O, const float* L, const void* dO, void* dQ, void* dK,
                          void* dV, void* workspace, size_t workspace_bytes, int B, int Hq,
                          int Hkv, int N, int d, int causal, float scale, void* stream) {
    return bwd_impl(false, stages, false, nullptr, Q, K, V, O, L, dO, dQ, dK, dV, workspace, workspace_bytes, B, Hq,
                    Hkv, N, d, causal, scale, stream);
}

fa2_status fa2_bwd_f16(const void* Q, const void* K, const void* V, const void* O, const float* L,
                       const void* dO, void* dQ, void* dK, void* dV, void* workspace,
                       size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, int causal,
                       float scale, void* stream) {
    return bwd_impl(true, FA2_BWD_ALL, false, nullptr, Q, K, V, O, L, dO, dQ, dK, dV, workspace, workspace_bytes,
                    B, Hq, Hkv, N, d, causal, scale, stream);
}

fa2_status fa2_bwd_stages_f16(unsigned stages, const void* Q, const void* K, const void* V,
                              const void* O, const float* L, const void* dO, void* dQ, void* dK,
                              void* dV, void* workspace, size_t workspace_bytes, int B, int Hq,
                              int Hkv, int N, int d, int causal, float scale, void* stream) {
    return bwd_impl(true, stages, false, nullptr, Q, K, V, O, L, dO, dQ, dK, dV, workspace, workspace_bytes, B, Hq,
                    Hkv, N, d, causal, scale, stream);
}

fa2_status fa2_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O,
                           const float* L, const void* dO, void* dQ, void* dK, void* dV, int B,
                           int Hq, int Hkv, int N, int d, int causal, float scale, void* stream) {
    g_last_error[0] = '\0';
    bool empty;
    Sizes sz;
    fa2_status s = validate_bwd(Q, K, V, O, L, dO, dQ, dK, dV, nullptr, 0, B, Hq, Hkv, N, d, scale,
                                false, &empty, &sz, /*static_ws=*/true);
    if (s != FA2_OK || empty) return s;
    const size_t need = workspace_layout(sz.rows_pad, sz.q_elems, false).total;
    if (need > kScratchBytes) {
        std::snprintf(g_last_error, sizeof g_last_error,
                      "problem needs %zu bytes of scratch; the static scratch holds %zu "
                      "(B * Hq * N rounded up to 64 rows per head must stay within %zu rows)",
                      need, kScratchBytes, kScratchBytes / 8);
        return FA2_ERR_UNSUPPORTED;
    }
    void* ws = nullptr;
    s = scratch_for_current_device(&ws);
    if (s != FA2_OK) return s;
    return bwd_impl(false, FA2_BWD_ALL, false, nullptr, Q, K, V, O, L, dO, dQ, dK, dV, ws,
                    kScratchBytes, B, Hq, Hkv, N, d, causal, scale, stream);
}

fa2_status fa2_fwd_olo(const void* Q, const void* K, const void* V, void* O, void* O_lo, float* L,
                       int B, int Hq, int Hkv, int N, int d, int causal, float scale, void* stream) {
    return fwd_impl(false, false, nullptr, Q, K, V, O, L, B, Hq, Hkv, N, d, causal, scale, stream,
                    true, O_lo);
}

fa2_status fa2_bwd_olo(const void* Q, const void* K, const void* V, const void* O, const void* O_lo,
                       const float* L, const void* dO, void* dQ, void* dK, void* dV, void* workspace,
                       size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, int causal,
                       float scale, void* stream) {
    return bwd_impl(false, FA2_BWD_ALL, false, nullptr, Q, K, V, O, L, dO, dQ, dK, dV, workspace,
                    workspace_bytes, B, Hq, Hkv, N, d, causal, scale, stream, true, O_lo);
}

fa2_status fa2_bwd_stages_olo(unsigned stages, const void* Q, const void* K, const void* V,
                              const void* O, const void* O_lo, const float* L, const void* dO,
                              void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                              int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                              void* stream) {
    return bwd_impl(false, stages, false, nullptr, Q, K, V, O, L, dO, dQ, dK, dV, workspace,
                    workspace_bytes, B, Hq, Hkv, N, d, causal, scale, stream, true, O_lo);
}

fa2_status fa2_fwd_block_sparse(const void* Q, const void* K, const void* V, void* O, float* L,
                                const unsigned char* block_mask, int B, int Hq, int Hkv, int N,
                                int d, int causal, float scale, void* stream) {
    return fwd_impl(false, true, block_mask, Q, K, V, O, L, B, Hq, Hkv, N, d, causal, scale, stream);
}

fa2_status fa2_bwd_block_sparse(const void* Q, const void* K, const void* V, const void* O,
                                const float* L, const void* dO, void* dQ, void* dK, void* dV,
                                const unsigned char* block_mask, void* workspace,
                                size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                                int causal, float scale, void* stream) {
    return bwd_impl(false, FA2_BWD_ALL, true, block_mask, Q, K, V, O, L, dO, dQ, dK, dV, workspace,
                    workspace_bytes, B, Hq, Hkv, N, d, causal, scale, stream);
}

fa2_status fa2_fwd_block_sparse_f16(const void* Q, const void* K, const void* V, void* O, float* L,
                                    const unsigned char* block_mask, int B, int Hq, int Hkv, int N,
                                    int d, int causal, float scale, void* stream) {
    return fwd_impl(true, true, block_mask, Q, K, V, O, L, B, Hq, Hkv, N, d, causal, scale, stream);
}

fa2_status fa2_bwd_block_sparse_f16(const void* Q, const void* K, const void* V, const void* O,
                                    const float* L, const void* dO, void* dQ, void* dK, void* dV,
                                    const unsigned char* block_mask, void* workspace,
                                    size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                                    int causal, float scale, void* stream) {
    return bwd_impl(true, FA2_BWD_ALL, true, block_mask, Q, K, V, O, L, dO, dQ, dK, dV, workspace,
                    workspace_bytes, B, Hq, Hkv, N, d, causal, scale, stream);
}

}  // extern "C"
