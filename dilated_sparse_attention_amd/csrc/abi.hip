// C ABI of the RAT+ hot path (declared in include/rat.h): host-side argument
// validation, workspace sizing, work scheduling and kernel launches.
// Validation never touches the HIP runtime, so every error code is returned
// before anything is enqueued.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "rat.h"
#include "rat_internal.h"
#include "rat_plan.h"

using namespace rat;

namespace {

thread_local int g_last_hip_error = 0;

rat_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return RAT_OK;
    g_last_hip_error = (int)e;
    return RAT_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t elem_size(rat_dtype t) { return t == RAT_DTYPE_F32 ? 4 : 2; }

bool dtype_ok(int t) { return t == RAT_DTYPE_F32 || t == RAT_DTYPE_BF16; }

bool d_ok(int d) { return d == 64 || d == 128; }

const int64_t kMaxElems = (int64_t)1 << 31;

// [B,T,H,d] (or any product of four positive ints) below 2^31 elements
bool size_ok(int64_t a, int64_t b, int64_t c, int64_t d)
{
    const int64_t n = a * b;
    if (n >= kMaxElems) return false;
    const int64_t n2 = n * c;
    if (n2 >= kMaxElems) return false;
    return n2 * d < kMaxElems;
}

// Decode caches: the kernels address them with 64-bit offsets, so only one
// head's rows (cap x d) and the B x H x d query rows need 32-bit indices.
bool caches_ok(int B, int H, int d, int nd_cap, int w_cap)
{
    return size_ok(B, H, d, 1) && (int64_t)nd_cap * d < kMaxElems && (int64_t)std::max(w_cap, 1) * d < kMaxElems;
}

ScanPlan scan_plan(int B, int T, int H, int d, int L, rat_dtype dtype)
{
    return rat::scan_plan(B, T, H, d, L, dtype == RAT_DTYPE_BF16);
}

// compute units of the current device (cached per device)
int device_cu_count()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

bool scan_uses_workspace(int T, int L, rat_recur_mode mode)
{
    return L >= T || mode == RAT_RECUR_RESTART;
}

// The scan after validation (workspace already checked).  hist: write the
// states as a per-residue history instead of [B][T][H][d].
rat_status run_scan(const void* k, const void* v, const void* g, void* ks, void* vs, int B, int T, int H, int d, int L,
             rat_recur_mode mode, rat_dtype dtype, void* workspace, float* final_state, const StateHist* hist,
             hipStream_t s)
{
    const bool bf16 = dtype == RAT_DTYPE_BF16;
    if (scan_uses_workspace(T, L, mode)) {
        const ScanPlan p = scan_plan(B, T, H, d, L, dtype);
        ScanFullArgs a;
        memset(&a, 0, sizeof(a));
        a.k = k; a.v = v; a.g = g; a.ks = ks; a.vs = vs;
        a.T = T; a.N = H * d; a.nblk = p.nblk; a.nseq = p.nseq; a.nchunk = p.nchunk;
        a.L = L >= T ? 0 : L; a.nwg = p.nwg;
        char* ws = static_cast<char*>(workspace);
        a.hdr = reinterpret_cast<ScanHeader*>(ws);
        a.agg = reinterpret_cast<uint64_t*>(ws + p.agg_off);
        a.incl = reinterpret_cast<uint64_t*>(ws + p.incl_off);
        a.fin = final_state;
        a.d = d;
        if (hist) a.hist = *hist;
        return hip_status(launch_scan_full(a, bf16, hist != nullptr, p.wide, s));
    }
    ScanSlideArgs a;
    memset(&a, 0, sizeof(a));
    a.k = k; a.v = v; a.g = g; a.ks = ks; a.vs = vs;
    a.B = B; a.T = T; a.N = H * d; a.L = L;
    if (hist) a.hist = *hist;
    if (bf16 && L == 64 && a.N % 64 == 0) return hip_status(launch_scan_slide64(a, hist != nullptr, s));
    const int ntiles = (T + L - 1) / L;
    // spans of at least 256 tokens: one halo tile per span
    a.tiles_per_span = std::max(1, (256 + L - 1) / L);
    const int nspans = (ntiles + a.tiles_per_span - 1) / a.tiles_per_span;
    const int cgroups = (a.N + 63) / 64;
    return hip_status(launch_scan_sliding(a, nspans * B * cgroups, bf16, hist != nullptr, s));
}


// Workspace of the backward: per query row (lse, delta) and its raw
// window's partial softmax sums, the state gradients, the per-chunk maps and
// carries; every part 256-byte aligned.
struct BwdPlan {
    int nchunk;
    size_t off_lse, off_delta, off_bstat, off_dks, off_dvs, off_maps, off_carry, bytes;
};

BwdPlan bwd_plan(int B, int T, int H, int d)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    BwdPlan p;
    p.nchunk = (T + kBwdChunk - 1) / kBwdChunk;
    const size_t rows = (size_t)B * T * H, elems = rows * d, cells = (size_t)p.nchunk * B * H * d;
    p.off_lse = 0;
    p.off_delta = up(p.off_lse + rows * 4);
    p.off_bstat = up(p.off_delta + rows * 4);
    p.off_dks = up(p.off_bstat + rows * 3 * 4);
    p.off_dvs = up(p.off_dks + elems * 4);
    p.off_maps = up(p.off_dvs + elems * 4);
    p.off_carry = up(p.off_maps + cells * 5 * 4);
    p.bytes = up(p.off_carry + cells * 4 * 4);
    return p;
}
}  // namespace

extern "C" {

const char* rat_status_string(rat_status s)
{
    switch (s) {
    case RAT_OK: return "ok";
    case RAT_ERR_NULL: return "a required pointer is NULL";
    case RAT_ERR_SHAPE: return "a size or per-head parameter is out of range";
    case RAT_ERR_UNSUPPORTED: return "valid arguments that this build does not support";
    case RAT_ERR_ALIAS: return "an output aliases an input";
    case RAT_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case RAT_ERR_HIP: return "a HIP launch failed";
    case RAT_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    default: return "unknown status";
    }
}

int rat_last_hip_error(void) { return g_last_hip_error; }

size_t rat_scan_workspace_bytes(int B, int T, int H, int d, int L, rat_recur_mode mode, rat_dtype dtype)
{
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || L < 1 || !dtype_ok(dtype)) return 0;
    if (!scan_uses_workspace(T, L, mode)) return 0;
    return scan_plan(B, T, H, d, L, dtype).bytes;
}

rat_status rat_scan_prefill(const void* k, const void* v, const void* gate_logits, void* k_state, void* v_state,
                     int B, int T, int H, int d, int L, rat_recur_mode mode, rat_dtype dtype,
                     void* workspace, size_t workspace_bytes, float* final_state, void* stream)
{
    if (!k || !v || !gate_logits || !k_state || !v_state) return RAT_ERR_NULL;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || L < 1) return RAT_ERR_SHAPE;
    if (mode != RAT_RECUR_RESTART && mode != RAT_RECUR_SLIDING) return RAT_ERR_SHAPE;
    if (!dtype_ok(dtype) || !d_ok(d) || !size_ok(B, T, H, d)) return RAT_ERR_UNSUPPORTED;
    if (mode == RAT_RECUR_SLIDING && L < T && L > 64) return RAT_ERR_UNSUPPORTED;
    const void* ins[3] = {k, v, gate_logits};
    for (const void* in : ins)
        if (in == k_state || in == v_state) return RAT_ERR_ALIAS;
    if (k_state == v_state) return RAT_ERR_ALIAS;
    const void* all[5] = {k, v, gate_logits, k_state, v_state};
    for (const void* p : all)
        if (!aligned16(p)) return RAT_ERR_ALIGN;
    if (final_state) {
        if (!scan_uses_workspace(T, L, mode)) return RAT_ERR_UNSUPPORTED;  // SLIDING keeps no single state
        for (const void* p : all)
            if (p == final_state) return RAT_ERR_ALIAS;
        if (!aligned16(final_state)) return RAT_ERR_ALIGN;
    }
    if (scan_uses_workspace(T, L, mode)) {
        const ScanPlan p = scan_plan(B, T, H, d, L, dtype);
        if (!workspace || workspace_bytes < p.bytes || ((uintptr_t)workspace & 255u)) return RAT_ERR_WORKSPACE;
    }
    return run_scan(k, v, gate_logits, k_state, v_state, B, T, H, d, L, mode, dtype, workspace, final_state,
                    nullptr, (hipStream_t)stream);
}

namespace {

rat_status check_heads(int H, const int* D, const int* W, bool* any_w)
{
    if (!D || !W) return RAT_ERR_NULL;
    if (H > kAttnMaxHeads) return RAT_ERR_UNSUPPORTED;
    *any_w = false;
    for (int h = 0; h < H; ++h) {
        if (D[h] < 1 || W[h] < 0) return RAT_ERR_SHAPE;
        if (W[h] > 0) *any_w = true;
    }
    return RAT_OK;
}

}  // namespace

size_t rat_attn_prefill_workspace_bytes(int B, int T, int H, int d, const int* D, const int* W, rat_dtype dtype)
{
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || !dtype_ok(dtype)) return 0;
    bool any_w = false;
    if (check_heads(H, D, W, &any_w) != RAT_OK || !any_w || dtype != RAT_DTYPE_BF16) return 0;
    return (size_t)B * T * H * 2 * sizeof(float);
}

namespace {

// bf16 prefill attention, relative dilation (chunk = 0) or chunk grid
// (chunk = 1: every head's W is 1 over the states, passed as k_raw / v_raw).
// Heads with W > 0 first get their raw-key band (one workgroup per 256
// contiguous queries), which leaves a partial softmax state per query in
// `out` and the workspace; then every head runs the persistent dilated
// kernel (items = (b, h, r, 256-row chunk)), which continues from those
// states.  Heads are grouped into (D, W) classes; classes with the longest
// single items come first, each class's levels most expensive first.
rat_status attn_prefill_bf16(const void* q, const void* k_state, const void* v_state, const void* k_raw,
                      const void* v_raw, void* out, int B, int T, int H, int d, const int* D, const int* W,
                      bool any_w, float scale, int chunk, int n_cap, void* workspace, size_t workspace_bytes,
                      hipStream_t s)
{
    if (any_w) {
        const size_t need = (size_t)B * T * H * 2 * sizeof(float);
        if (!workspace || workspace_bytes < need || !aligned16(workspace)) return RAT_ERR_WORKSPACE;
    }
    AttnArgs lng, sht, band;
    memset(&lng, 0, sizeof(lng));
    lng.q = q; lng.ks = k_state; lng.vs = v_state; lng.kr = k_raw; lng.vr = v_raw; lng.out = out;
    lng.ml = static_cast<float*>(workspace);
    sht = lng;
    if (!attn_launch_plans(B, T, H, D, W, scale, chunk, n_cap, lng, sht, band)) return RAT_ERR_UNSUPPORTED;
    // the band pass first: windowed classes continue from its partial
    // state.  Long residues: one eight-wave workgroup per CU; the band and
    // short residues: two four-wave workgroups per CU.
    const int cu = device_cu_count();
    if (band.nblocks > 0) {
        const rat_status rc = hip_status(launch_attn_band_bf16(band, d, std::min(band.nblocks, 2 * cu), s));
        if (rc != RAT_OK) return rc;
    }
    if (lng.nblocks > 0) {
        const rat_status rc = hip_status(launch_attn_dilated_bf16(lng, d, std::min(lng.nblocks, cu), s));
        if (rc != RAT_OK) return rc;
    }
    if (sht.nblocks > 0) return hip_status(launch_attn_dilated_bf16(sht, d, std::min(sht.nblocks, 2 * cu), s));
    return RAT_OK;
}

}  // namespace

rat_status rat_dilated_attn_prefill(const void* q, const void* k_state, const void* v_state, const void* k_raw,
                             const void* v_raw, void* out, int B, int T, int H, int d, const int* D, const int* W,
                             float scale, rat_dtype dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!q || !k_state || !v_state || !out) return RAT_ERR_NULL;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0) return RAT_ERR_SHAPE;
    bool any_w = false;
    const rat_status hc = check_heads(H, D, W, &any_w);
    if (hc != RAT_OK) return hc;
    if (any_w && (!k_raw || !v_raw)) return RAT_ERR_NULL;
    if (!dtype_ok(dtype) || !d_ok(d) || !size_ok(B, T, H, d)) return RAT_ERR_UNSUPPORTED;
    if (!(scale == scale)) return RAT_ERR_SHAPE;
    const void* ins[5] = {q, k_state, v_state, k_raw, v_raw};
    for (const void* in : ins)
        if (in && in == out) return RAT_ERR_ALIAS;
    for (const void* p : ins)
        if (p && !aligned16(p)) return RAT_ERR_ALIGN;
    if (!aligned16(out)) return RAT_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;

    if (dtype == RAT_DTYPE_F32) {
        AttnF32Args a;
        memset(&a, 0, sizeof(a));
        a.q = (const float*)q; a.ks = (const float*)k_state; a.vs = (const float*)v_state;
        a.kr = (const float*)k_raw; a.vr = (const float*)v_raw; a.out = (float*)out;
        a.B = B; a.T = T; a.H = H; a.d = d; a.scale = scale;
        for (int h = 0; h < H; ++h) { a.D[h] = D[h]; a.W[h] = W[h]; }
        return hip_status(launch_attn_prefill_f32(a, s));
    }

    return attn_prefill_bf16(q, k_state, v_state, k_raw, v_raw, out, B, T, H, d, D, W, any_w, scale, 0, 0,
                             workspace, workspace_bytes, s);
}

rat_status rat_chunk_attn_prefill(const void* q, const void* k_state, const void* v_state, void* out, int B, int T, int H,
                           int d, const int* D, float scale, rat_dtype dtype, void* stream)
{
    if (!q || !k_state || !v_state || !out || !D) return RAT_ERR_NULL;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0) return RAT_ERR_SHAPE;
    if (H > kAttnMaxHeads) return RAT_ERR_UNSUPPORTED;
    int W0[kAttnMaxHeads];
    for (int h = 0; h < H; ++h) {
        if (D[h] < 1) return RAT_ERR_SHAPE;
        W0[h] = 0;
    }
    if (!dtype_ok(dtype) || !d_ok(d) || !size_ok(B, T, H, d)) return RAT_ERR_UNSUPPORTED;
    if (!(scale == scale)) return RAT_ERR_SHAPE;
    const void* ins[3] = {q, k_state, v_state};
    for (const void* in : ins)
        if (in == out) return RAT_ERR_ALIAS;
    for (const void* p : ins)
        if (!aligned16(p)) return RAT_ERR_ALIGN;
    if (!aligned16(out)) return RAT_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == RAT_DTYPE_F32) {
        AttnF32Args a;
        memset(&a, 0, sizeof(a));
        a.q = (const float*)q; a.ks = (const float*)k_state; a.vs = (const float*)v_state;
        a.out = (float*)out;
        a.B = B; a.T = T; a.H = H; a.d = d; a.scale = scale; a.chunk = 1;
        for (int h = 0; h < H; ++h) { a.D[h] = D[h]; a.W[h] = 0; }
        return hip_status(launch_attn_prefill_f32(a, s));
    }
    // dilated items whose keys are the chunk ends (residue D - 1) strictly
    // before each query, their softmax started from the query's own state
    return attn_prefill_bf16(q, k_state, v_state, nullptr, nullptr, out, B, T, H, d, D, W0, false, scale, 1, 0,
                             nullptr, 0, s);
}

namespace {

int decode_nsplit(int B, int H, int T, const int* D, const int* W)
{
    int nmax = 1;
    for (int h = 0; h < H; ++h) nmax = std::max(nmax, (T - 1) / D[h] + 1 + std::min(W[h], T));
    const int bh = B * H;
    const int want = (512 + bh - 1) / bh;          // aim at >= 512 workgroups
    const int cap = std::max(1, nmax / 256);        // at least 256 keys per split
    return std::max(1, std::min(want, cap));
}

}  // namespace

size_t rat_decode_workspace_bytes(int B, int H, int d, int T, const int* D, const int* W)
{
    if (B <= 0 || H <= 0 || d <= 0 || T <= 0 || !D || !W || H > kAttnMaxHeads) return 0;
    for (int h = 0; h < H; ++h)
        if (D[h] < 1 || W[h] < 0) return 0;
    const int ns = decode_nsplit(B, H, T, D, W);
    if (ns == 1) return 0;
    return (size_t)B * H * ns * (d + 2) * sizeof(float);
}

rat_status rat_layer_prefill(const void* q, const void* k, const void* v, const void* gate_logits, void* out, void* kc,
                      void* vc, int n_cap, void* kw, void* vw, int w_cap, float* final_state, int B, int T, int H,
                      int d, int L, rat_recur_mode mode, const int* D, const int* W, float scale, rat_dtype dtype,
                      void* scan_workspace, size_t scan_workspace_bytes, void* attn_workspace,
                      size_t attn_workspace_bytes, void* stream)
{
    if (!q || !k || !v || !gate_logits || !out || !kc || !vc) return RAT_ERR_NULL;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || L < 1 || n_cap <= 0 || w_cap < 0) return RAT_ERR_SHAPE;
    if (mode != RAT_RECUR_RESTART && mode != RAT_RECUR_SLIDING) return RAT_ERR_SHAPE;
    bool any_w = false;
    const rat_status hc = check_heads(H, D, W, &any_w);
    if (hc != RAT_OK) return hc;
    if (any_w && (!kw || !vw)) return RAT_ERR_NULL;
    for (int h = 0; h < H; ++h) {
        if ((T - 1) / D[h] >= n_cap / D[h]) return RAT_ERR_SHAPE;  // history rows of position T-1
        if (W[h] > w_cap) return RAT_ERR_SHAPE;                   // ring slots p mod W
    }
    if (!dtype_ok(dtype) || !d_ok(d) || !size_ok(B, T, H, d) || !size_ok(B, H, n_cap, d) ||
        !size_ok(B, H, std::max(w_cap, 1), d))
        return RAT_ERR_UNSUPPORTED;
    if (mode == RAT_RECUR_SLIDING && L < T && L > 64) return RAT_ERR_UNSUPPORTED;
    if (final_state && !scan_uses_workspace(T, L, mode)) return RAT_ERR_UNSUPPORTED;  // SLIDING: no single state
    if (!(scale == scale)) return RAT_ERR_SHAPE;
    const void* ins[4] = {q, k, v, gate_logits};
    const void* outs[6] = {out, kc, vc, kw, vw, final_state};
    for (int i = 0; i < 6; ++i) {
        if (!outs[i]) continue;
        for (const void* in : ins)
            if (outs[i] == in) return RAT_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (outs[j] == outs[i]) return RAT_ERR_ALIAS;
    }
    for (const void* x : ins)
        if (!aligned16(x)) return RAT_ERR_ALIGN;
    for (const void* x : outs)
        if (x && !aligned16(x)) return RAT_ERR_ALIGN;
    if (scan_uses_workspace(T, L, mode)) {
        const ScanPlan p = scan_plan(B, T, H, d, L, dtype);
        if (!scan_workspace || scan_workspace_bytes < p.bytes || ((uintptr_t)scan_workspace & 255u))
            return RAT_ERR_WORKSPACE;
    }
    const bool bf16 = dtype == RAT_DTYPE_BF16;
    if (bf16 && any_w) {
        const size_t need = (size_t)B * T * H * 2 * sizeof(float);
        if (!attn_workspace || attn_workspace_bytes < need || !aligned16(attn_workspace)) return RAT_ERR_WORKSPACE;
    }
    hipStream_t s = (hipStream_t)stream;

    // 1. the recurrence, its states written straight into the history
    StateHist hist;
    memset(&hist, 0, sizeof(hist));
    hist.n_cap = n_cap; hist.d = d; hist.H = H;
    for (int h = 0; h < H; ++h) hist.D[h] = D[h];
    rat_status rc = run_scan(k, v, gate_logits, kc, vc, B, T, H, d, L, mode, dtype, scan_workspace, final_state, &hist, s);
    if (rc != RAT_OK) return rc;
    // 2. the raw ring of the last W tokens
    if (any_w) {
        RingFillArgs r;
        memset(&r, 0, sizeof(r));
        r.k = k; r.v = v; r.kw = kw; r.vw = vw;
        r.B = B; r.T = T; r.H = H; r.d = d; r.w_cap = w_cap;
        for (int h = 0; h < H; ++h) r.W[h] = W[h];
        rc = hip_status(launch_ring_fill(r, bf16, s));
        if (rc != RAT_OK) return rc;
    }
    // 3. dilated (+ local window) attention over the history
    if (!bf16) {
        AttnF32Args a;
        memset(&a, 0, sizeof(a));
        a.q = (const float*)q; a.ks = (const float*)kc; a.vs = (const float*)vc;
        a.kr = (const float*)k; a.vr = (const float*)v; a.out = (float*)out;
        a.B = B; a.T = T; a.H = H; a.d = d; a.scale = scale; a.n_cap = n_cap;
        for (int h = 0; h < H; ++h) { a.D[h] = D[h]; a.W[h] = W[h]; }
        return hip_status(launch_attn_prefill_f32(a, s));
    }
    return attn_prefill_bf16(q, kc, vc, k, v, out, B, T, H, d, D, W, any_w, scale, 0, n_cap, attn_workspace,
                             attn_workspace_bytes, s);
}

rat_status rat_build_decode_caches(const void* k_state, const void* v_state, const void* k, const void* v, void* kc,
                            void* vc, int n_cap, void* kw, void* vw, int w_cap, int B, int T, int H, int d,
                            const int* D, const int* W, rat_dtype dtype, void* stream)
{
    if (!k_state || !v_state || !kc || !vc) return RAT_ERR_NULL;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || n_cap <= 0 || w_cap < 0) return RAT_ERR_SHAPE;
    bool any_w = false;
    const rat_status hc = check_heads(H, D, W, &any_w);
    if (hc != RAT_OK) return hc;
    if (any_w && (!k || !v || !kw || !vw)) return RAT_ERR_NULL;
    for (int h = 0; h < H; ++h) {
        if ((T - 1) / D[h] >= n_cap / D[h]) return RAT_ERR_SHAPE;  // history rows of position T-1
        if (W[h] > w_cap) return RAT_ERR_SHAPE;                   // ring slots p mod W
    }
    if (!dtype_ok(dtype) || !d_ok(d) || !size_ok(B, T, H, d) || !caches_ok(B, H, d, n_cap, w_cap))
        return RAT_ERR_UNSUPPORTED;
    const void* ins[4] = {k_state, v_state, k, v};
    const void* outs[4] = {kc, vc, kw, vw};
    for (int i = 0; i < 4; ++i) {
        if (!outs[i]) continue;
        for (const void* x : ins)
            if (x && x == outs[i]) return RAT_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (outs[j] == outs[i]) return RAT_ERR_ALIAS;
    }
    for (const void* x : ins)
        if (x && !aligned16(x)) return RAT_ERR_ALIGN;
    for (const void* x : outs)
        if (x && !aligned16(x)) return RAT_ERR_ALIGN;
    CacheArgs a;
    memset(&a, 0, sizeof(a));
    a.ks = k_state; a.vs = v_state; a.k = k; a.v = v; a.kc = kc; a.vc = vc; a.kw = kw; a.vw = vw;
    a.B = B; a.T = T; a.H = H; a.d = d; a.n_cap = n_cap; a.w_cap = w_cap;
    for (int h = 0; h < H; ++h) { a.D[h] = D[h]; a.W[h] = W[h]; }
    return hip_status(launch_cache_build(a, dtype == RAT_DTYPE_BF16, (hipStream_t)stream));
}

size_t rat_layer_backward_workspace_bytes(int B, int T, int H, int d)
{
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || !size_ok(B, T, H, d)) return 0;
    return bwd_plan(B, T, H, d).bytes;
}

rat_status rat_layer_backward(const void* q, const void* k, const void* v, const void* gate_logits, const void* k_state,
                       const void* v_state, const void* dout, float* dq, float* dk, float* dv, float* dgate, int B,
                       int T, int H, int d, int L, rat_recur_mode mode, const int* D, const int* W, float scale,
                       rat_dtype dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    const void* ins[7] = {q, k, v, gate_logits, k_state, v_state, dout};
    const void* outs[4] = {dq, dk, dv, dgate};
    for (const void* x : ins)
        if (!x) return RAT_ERR_NULL;
    for (const void* x : outs)
        if (!x) return RAT_ERR_NULL;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || L < 1) return RAT_ERR_SHAPE;
    if (mode != RAT_RECUR_RESTART && mode != RAT_RECUR_SLIDING) return RAT_ERR_SHAPE;
    bool any_w = false;
    const rat_status hc = check_heads(H, D, W, &any_w);
    if (hc != RAT_OK) return hc;
    if (!dtype_ok(dtype) || !d_ok(d) || !size_ok(B, T, H, d)) return RAT_ERR_UNSUPPORTED;
    if (!(scale == scale)) return RAT_ERR_SHAPE;
    for (int i = 0; i < 4; ++i) {
        for (const void* x : ins)
            if (outs[i] == x) return RAT_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (outs[j] == outs[i]) return RAT_ERR_ALIAS;
    }
    for (const void* x : ins)
        if (!aligned16(x)) return RAT_ERR_ALIGN;
    for (const void* x : outs)
        if (!aligned16(x)) return RAT_ERR_ALIGN;
    const BwdPlan p = bwd_plan(B, T, H, d);
    if (!workspace || workspace_bytes < p.bytes || ((uintptr_t)workspace & 255u)) return RAT_ERR_WORKSPACE;

    BwdArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q; a.k = k; a.v = v; a.g = gate_logits; a.ks = k_state; a.vs = v_state; a.dout = dout;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dgate;
    char* ws = static_cast<char*>(workspace);
    a.lse = reinterpret_cast<float*>(ws + p.off_lse);
    a.delta = reinterpret_cast<float*>(ws + p.off_delta);
    a.dks = reinterpret_cast<float*>(ws + p.off_dks);
    a.dvs = reinterpret_cast<float*>(ws + p.off_dvs);
    a.maps = reinterpret_cast<float*>(ws + p.off_maps);
    a.carry = reinterpret_cast<float*>(ws + p.off_carry);
    a.bstat = reinterpret_cast<float*>(ws + p.off_bstat);
    a.B = B; a.T = T; a.H = H; a.d = d;
    a.sliding = (mode == RAT_RECUR_SLIDING && L < T) ? 1 : 0;
    a.L = L >= T ? 0 : L;  // the RESTART period, or the SLIDING window
    a.nchunk = p.nchunk;
    a.scale = scale;
    a.mfma = dtype == RAT_DTYPE_BF16 ? 1 : 0;
    a.raw = (any_w || !a.mfma) ? 1 : 0;
    int64_t items = 0;
    for (int h = 0; h < H; ++h) {
        a.D[h] = D[h];
        a.W[h] = W[h];
        a.mitem[h] = (int)items;
        if (a.mfma) {
            // B x min(D, T) residues x blocks of 16 kBwdWaves rows of the longest residue
            const int64_t nb = ((T + D[h] - 1) / D[h] + 16 * kBwdWaves - 1) / (16 * kBwdWaves);
            items += (int64_t)B * std::min(D[h], T) * nb;
        }
        if (items >= ((int64_t)1 << 31)) return RAT_ERR_UNSUPPORTED;
    }
    a.mitem[H] = (int)items;
    // the band passes: one item per (head, batch, block of 16 kBwdWaves positions)
    if (a.mfma && any_w && (int64_t)H * B * ((T + 16 * kBwdWaves - 1) / (16 * kBwdWaves)) >= ((int64_t)1 << 31))
        return RAT_ERR_UNSUPPORTED;
    return hip_status(launch_backward(a, dtype == RAT_DTYPE_BF16, (hipStream_t)stream));
}

namespace {

// Validation shared by the decode entry points; on success *ns holds the
// key-range splits and *need the bytes of split partials they use.
rat_status check_decode(const void* q, const void* kd, const void* vd, int nd_cap, const void* kw, const void* vw,
                        int w_cap, void* out, int B, int T, int H, int d, const int* D, const int* W, float scale,
                        rat_dtype dtype, int* ns, size_t* need)
{
    if (!q || !kd || !vd || !out) return RAT_ERR_NULL;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || nd_cap <= 0 || w_cap < 0) return RAT_ERR_SHAPE;
    bool any_w = false;
    const rat_status hc = check_heads(H, D, W, &any_w);
    if (hc != RAT_OK) return hc;
    if (any_w && (!kw || !vw)) return RAT_ERR_NULL;
    for (int h = 0; h < H; ++h) {
        if ((T - 1) / D[h] + 1 > nd_cap) return RAT_ERR_SHAPE;
        if (std::min(W[h], T) > w_cap) return RAT_ERR_SHAPE;
    }
    if (!dtype_ok(dtype) || !d_ok(d) || !caches_ok(B, H, d, nd_cap, w_cap))
        return RAT_ERR_UNSUPPORTED;
    if (!(scale == scale)) return RAT_ERR_SHAPE;
    const void* ins[5] = {q, kd, vd, kw, vw};
    for (const void* in : ins)
        if (in && in == out) return RAT_ERR_ALIAS;
    for (const void* p : ins)
        if (p && !aligned16(p)) return RAT_ERR_ALIGN;
    if (!aligned16(out)) return RAT_ERR_ALIGN;
    *ns = decode_nsplit(B, H, T, D, W);
    *need = *ns == 1 ? 0 : (size_t)B * H * *ns * (d + 2) * sizeof(float);
    return RAT_OK;
}

rat_status launch_decode_checked(const void* q, const void* kd, const void* vd, int nd_cap, const void* kw,
                                 const void* vw, int w_cap, void* out, int B, int T, int H, int d, const int* D,
                                 const int* W, float scale, rat_dtype dtype, int ns, float* part, hipStream_t s)
{
    DecodeArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q; a.kd = kd; a.vd = vd; a.kw = kw ? kw : kd; a.vw = vw ? vw : vd; a.out = out;
    a.part = part;
    a.B = B; a.H = H; a.T = T; a.nd_cap = nd_cap; a.w_cap = w_cap; a.nsplit = ns;
    a.scale_log2 = scale * 1.4426950408889634f;
    for (int h = 0; h < H; ++h) { a.D[h] = D[h]; a.W[h] = W[h]; }
    return hip_status(launch_decode(a, d, dtype == RAT_DTYPE_BF16, s));
}

}  // namespace

rat_status rat_dilated_attn_decode(const void* q, const void* kd, const void* vd, int nd_cap, const void* kw, const void* vw,
                            int w_cap, void* out, int B, int T, int H, int d, const int* D, const int* W, float scale,
                            rat_dtype dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    int ns = 1;
    size_t need = 0;
    const rat_status rc = check_decode(q, kd, vd, nd_cap, kw, vw, w_cap, out, B, T, H, d, D, W, scale, dtype, &ns,
                                       &need);
    if (rc != RAT_OK) return rc;
    if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))) return RAT_ERR_WORKSPACE;
    return launch_decode_checked(q, kd, vd, nd_cap, kw, vw, w_cap, out, B, T, H, d, D, W, scale, dtype, ns,
                                 static_cast<float*>(workspace), (hipStream_t)stream);
}

size_t rat_decode_static_scratch_bytes(void) { return kDecodeScratchBytes; }

rat_status rat_dilated_attn_decode_static(const void* q, const void* kd, const void* vd, int nd_cap, const void* kw,
                                          const void* vw, int w_cap, void* out, int B, int T, int H, int d,
                                          const int* D, const int* W, float scale, rat_dtype dtype, void* stream)
{
    int ns = 1;
    size_t need = 0;
    const rat_status rc = check_decode(q, kd, vd, nd_cap, kw, vw, w_cap, out, B, T, H, d, D, W, scale, dtype, &ns,
                                       &need);
    if (rc != RAT_OK) return rc;
    if (need > kDecodeScratchBytes) return RAT_ERR_WORKSPACE;
    float* part = nullptr;
    if (need > 0) {
        void* p = nullptr;
        const hipError_t e = decode_scratch(&p);
        if (e != hipSuccess) return hip_status(e);
        part = static_cast<float*>(p);
    }
    return launch_decode_checked(q, kd, vd, nd_cap, kw, vw, w_cap, out, B, T, H, d, D, W, scale, dtype, ns, part,
                                 (hipStream_t)stream);
}

rat_status rat_decode_step(const void* q, const void* k_new, const void* v_new, const void* gate_new, float* state,
                    void* kc, void* vc, int n_cap, void* kw, void* vw, int w_cap, void* out, int B, int T, int H,
                    int d, int L, const int* D, const int* W, float scale, rat_dtype dtype, void* workspace,
                    size_t workspace_bytes, void* stream)
{
    if (!q || !k_new || !v_new || !gate_new || !state || !kc || !vc || !out) return RAT_ERR_NULL;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || n_cap <= 0 || w_cap < 0 || L < 1) return RAT_ERR_SHAPE;
    bool any_w = false;
    const rat_status hc = check_heads(H, D, W, &any_w);
    if (hc != RAT_OK) return hc;
    if (any_w && (!kw || !vw)) return RAT_ERR_NULL;
    const int p = T - 1;  // position of the new token
    for (int h = 0; h < H; ++h) {
        if (p / D[h] >= n_cap / D[h]) return RAT_ERR_SHAPE;  // history rows of the residue
        if (W[h] > w_cap) return RAT_ERR_SHAPE;               // ring slot p mod W
    }
    if (!dtype_ok(dtype) || !d_ok(d) || !caches_ok(B, H, d, n_cap, w_cap))
        return RAT_ERR_UNSUPPORTED;
    if (!(scale == scale)) return RAT_ERR_SHAPE;
    const void* ins[5] = {q, k_new, v_new, gate_new, state};
    const void* outs[5] = {kc, vc, kw, vw, out};
    for (const void* o : outs)
        for (const void* in : ins)
            if (o && o == in) return RAT_ERR_ALIAS;
    if (kc == vc || (kw && (kw == vw || kw == kc || kw == vc)) || out == kc || out == vc) return RAT_ERR_ALIAS;
    for (const void* x : ins)
        if (!aligned16(x)) return RAT_ERR_ALIGN;
    for (const void* x : outs)
        if (x && !aligned16(x)) return RAT_ERR_ALIGN;
    const int ns = decode_nsplit(B, H, T, D, W);
    const size_t need = ns == 1 ? 0 : (size_t)B * H * ns * (d + 2) * sizeof(float);
    if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))) return RAT_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const bool bf16 = dtype == RAT_DTYPE_BF16;

    StepArgs st;
    memset(&st, 0, sizeof(st));
    st.k_new = k_new; st.v_new = v_new; st.g_new = gate_new; st.state = state;
    st.kc = kc; st.vc = vc; st.kw = kw; st.vw = vw;
    st.B = B; st.H = H; st.d = d; st.n_cap = n_cap; st.w_cap = w_cap;
    st.restart = (L < T && p % L == 0) ? 1 : 0;
    DecodeArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q; a.kd = kc; a.vd = vc; a.kw = kw ? kw : kc; a.vw = vw ? vw : vc; a.out = out;
    a.part = static_cast<float*>(workspace);
    a.B = B; a.H = H; a.T = T; a.nd_cap = n_cap; a.w_cap = w_cap; a.nsplit = ns;
    a.scale_log2 = scale * 1.4426950408889634f;
    for (int h = 0; h < H; ++h) {
        const int mcap = n_cap / D[h];
        st.slot_c[h] = (p % D[h]) * mcap + p / D[h];
        st.slot_w[h] = W[h] > 0 ? p % W[h] : -1;
        a.D[h] = D[h]; a.W[h] = W[h];
        a.dil_off[h] = (p % D[h]) * mcap;
    }
    const rat_status rc = hip_status(launch_decode_step(st, bf16, s));
    if (rc != RAT_OK) return rc;
    return hip_status(launch_decode(a, d, bf16, s));
}

// Longest recurrence window a SLIDING decode step runs over (each step
// reads the window's L raw rows).
constexpr int kSlideDecodeMaxL = 1024;

rat_status rat_decode_step_sliding(const void* q, const void* k_new, const void* v_new, const void* gate_new,
                                   void* rk, void* rv, void* rg, int L, void* kc, void* vc, int n_cap, void* kw,
                                   void* vw, int w_cap, void* out, int B, int T, int H, int d, const int* D,
                                   const int* W, float scale, rat_dtype dtype, void* workspace,
                                   size_t workspace_bytes, void* stream)
{
    if (!q || !k_new || !v_new || !gate_new || !rk || !rv || !rg || !kc || !vc || !out) return RAT_ERR_NULL;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || n_cap <= 0 || w_cap < 0 || L < 1) return RAT_ERR_SHAPE;
    bool any_w = false;
    const rat_status hc = check_heads(H, D, W, &any_w);
    if (hc != RAT_OK) return hc;
    if (any_w && (!kw || !vw)) return RAT_ERR_NULL;
    const int p = T - 1;  // position of the new token
    for (int h = 0; h < H; ++h) {
        if (p / D[h] >= n_cap / D[h]) return RAT_ERR_SHAPE;  // history rows of the residue
        if (W[h] > w_cap) return RAT_ERR_SHAPE;               // ring slot p mod W
    }
    if (L > kSlideDecodeMaxL) return RAT_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype) || !d_ok(d) || !caches_ok(B, H, d, n_cap, w_cap) || !caches_ok(B, H, d, L, 0))
        return RAT_ERR_UNSUPPORTED;
    if (!(scale == scale)) return RAT_ERR_SHAPE;
    const void* ins[4] = {q, k_new, v_new, gate_new};
    const void* outs[8] = {rk, rv, rg, kc, vc, kw, vw, out};
    for (int i = 0; i < 8; ++i) {
        if (!outs[i]) continue;
        for (const void* in : ins)
            if (outs[i] == in) return RAT_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (outs[j] == outs[i]) return RAT_ERR_ALIAS;
    }
    for (const void* x : ins)
        if (!aligned16(x)) return RAT_ERR_ALIGN;
    for (const void* x : outs)
        if (x && !aligned16(x)) return RAT_ERR_ALIGN;
    const int ns = decode_nsplit(B, H, T, D, W);
    const size_t need = ns == 1 ? 0 : (size_t)B * H * ns * (d + 2) * sizeof(float);
    if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))) return RAT_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const bool bf16 = dtype == RAT_DTYPE_BF16;

    SlideStepArgs st;
    memset(&st, 0, sizeof(st));
    st.k_new = k_new; st.v_new = v_new; st.g_new = gate_new;
    st.rk = rk; st.rv = rv; st.rg = rg;
    st.kc = kc; st.vc = vc; st.kw = kw; st.vw = vw;
    st.B = B; st.H = H; st.d = d; st.n_cap = n_cap; st.w_cap = w_cap; st.L = L; st.p = p;
    for (int h = 0; h < H; ++h) {
        st.slot_c[h] = (p % D[h]) * (n_cap / D[h]) + p / D[h];
        st.slot_w[h] = W[h] > 0 ? p % W[h] : -1;
    }
    const rat_status rc = hip_status(launch_decode_step_sliding(st, bf16, s));
    if (rc != RAT_OK) return rc;
    DecodeArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q; a.kd = kc; a.vd = vc; a.kw = kw ? kw : kc; a.vw = vw ? vw : vc; a.out = out;
    a.part = static_cast<float*>(workspace);
    a.B = B; a.H = H; a.T = T; a.nd_cap = n_cap; a.w_cap = w_cap; a.nsplit = ns;
    a.scale_log2 = scale * 1.4426950408889634f;
    for (int h = 0; h < H; ++h) {
        a.D[h] = D[h]; a.W[h] = W[h];
        a.dil_off[h] = (p % D[h]) * (n_cap / D[h]);
    }
    return hip_status(launch_decode(a, d, bf16, s));
}

rat_status rat_sliding_state_from_prefill(const void* k, const void* v, const void* gate_logits, void* rk, void* rv,
                                          void* rg, int B, int T, int H, int d, int L, rat_dtype dtype,
                                          void* stream)
{
    if (!k || !v || !gate_logits || !rk || !rv || !rg) return RAT_ERR_NULL;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || L < 1) return RAT_ERR_SHAPE;
    if (L > kSlideDecodeMaxL) return RAT_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype) || !d_ok(d) || !size_ok(B, T, H, d) || !caches_ok(B, H, d, L, 0))
        return RAT_ERR_UNSUPPORTED;
    const void* ins[3] = {k, v, gate_logits};
    const void* outs[3] = {rk, rv, rg};
    for (int i = 0; i < 3; ++i) {
        for (const void* in : ins)
            if (outs[i] == in) return RAT_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (outs[j] == outs[i]) return RAT_ERR_ALIAS;
    }
    for (const void* x : ins)
        if (!aligned16(x)) return RAT_ERR_ALIGN;
    for (const void* x : outs)
        if (!aligned16(x)) return RAT_ERR_ALIGN;
    SlideFillArgs a;
    memset(&a, 0, sizeof(a));
    a.k = k; a.v = v; a.g = gate_logits; a.rk = rk; a.rv = rv; a.rg = rg;
    a.B = B; a.T = T; a.H = H; a.d = d; a.L = L;
    return hip_status(launch_sliding_fill(a, dtype == RAT_DTYPE_BF16, (hipStream_t)stream));
}

}  // extern "C"
