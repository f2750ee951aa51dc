// C-ABI entry points of libssm, the chunk-carry combine and the empty-sequence fill.
//
// Long sequences are cut into chunks: a carry pass stores, per chunk and state,
// the chunk's decay P (the product of A_bar over the chunk: exp(A sum delta)
// for the exponential discretisations) and the end state H from h = 0; the
// combine folds them in order with (P1, H1) o (P2, H2) = (P2 P1, P2 H1 + H2) (skill page
// "State Space Models Mamba", section "Hardware-Efficient Scan": the
// recurrence is linear, so it admits an associative scan); a second scan pass
// then starts every chunk from its carried-in state.
#include "ssm_device.h"

#include <mutex>

namespace ssm {

hipError_t launch_status(hipStream_t s) {
    static const bool sync = env_flag("SSM_SYNC");
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && sync) e = hipStreamSynchronize(s);
    return e;
}

namespace {

// Carries of the carry pass, folded in sequence order with a parallel scan (segment_scan in
// ssm_device.h): one segment of S
// lanes per (b, d, n), lane j holding chunk t + j of a tile of S chunks (padded with the
// identity (1, 0)); the state entering the tile is the carry.
//   h_in(0) = h0,  h_in(c+1) = P_c * h_in(c) + H_c
// overwrites slot c with h_in(c+1), the state chunk c+1 starts from.
template <int S>
__global__ void __launch_bounds__(256) combine_kernel(ScanArgs a) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t DN = a.D * a.N;
    const int64_t item = gid / S;   // (b, d, n)
    const int j = static_cast<int>(gid % S);
    const bool ok = item < a.B * DN;
    const int64_t b = ok ? item / DN : 0, dn = ok ? item % DN : 0;
    const int64_t C1 = a.n_chunks - 1;
    float carry = (ok && a.h0) ? a.h0[item] : 0.0f;
    for (int64_t t = 0; t < C1; t += S) {
        const int64_t c = t + j;
        const bool v = ok && c < C1;
        const int64_t at = (b * C1 + c) * DN + dn;
        float P = v ? a.ws_P[at] : 1.0f, H = v ? a.ws_H[at] : 0.0f;
        segment_scan<S>(P, H);
        const float hin = __builtin_fmaf(P, carry, H);
        if (v) a.ws_H[at] = hin;
        carry = __shfl(hin, S - 1, S);
    }
}

// Carries of the local scans (every chunk scanned from its own start, ScanArgs::ws_Hl and
// the delta sums S_part): chunk c's decay is P_c = exp(A sum of its delta); chunk 0 starts
// from h0, so its end state is exact and P_0 = 0.  The scan gives each chunk c >= 1 its
// carried-in state h_in(c) (into ws_H) and the last chunk's true end state (h_last).  It also
// decides whether the carried-in state still matters after the prefix that the rescan
// covers: the part of chunk c's state that comes from h_in decays as exp(A * cumulative
// delta), so after the first y_skip steps it is h_in * exp(A * S_pre) and keeps shrinking
// when A <= 0.  Below 2^-100 its share of any output is far under fp32 resolution; otherwise
// (or when A > 0) the chunk's flag is set and the rest of the chunk is rescanned too.
template <int S>
__global__ void __launch_bounds__(256) local_combine_kernel(ScanArgs a, float *h_last) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t D = a.D, N = a.N, DN = D * N, C = a.n_chunks;
    const int64_t item = gid / S;   // (b, d, n)
    const int j = static_cast<int>(gid % S);
    const bool ok = item < a.B * DN;
    const int64_t b = ok ? item / DN : 0, dn = ok ? item % DN : 0;
    const int64_t d = dn / N;
    const float Av = ok ? a.A[dn] : 0.0f;
    const float al = Av * kLog2e;
    constexpr float kNegligible = 7.888609052210118e-31f;   // 2^-100
    float carry = 0.0f;
    for (int64_t t = 0; t < C; t += S) {
        const int64_t c = t + j;
        const bool v = ok && c < C;
        float sf = 0.0f, sp = 0.0f;
        if (v) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                sf += a.S_part[((b * C + c) * 8 + r) * D + d];
                sp += a.S_part[(((a.B + b) * C + c) * 8 + r) * D + d];
            }
        }
        float P = v ? (c == 0 ? 0.0f : __builtin_amdgcn_exp2f(al * sf)) : 1.0f;
        float H = v ? a.ws_Hl[(b * C + c) * DN + dn] : 0.0f;
        segment_scan<S>(P, H);
        const float hend = __builtin_fmaf(P, carry, H);   // chunk c's true end state
        float hin = __shfl_up(hend, 1, S);                 // chunk c's start state
        if (j == 0) hin = carry;
        if (v && c >= 1) {
            a.ws_H[((b * (C - 1) + (c - 1)) * DN) + dn] = hin;
            const float g = __builtin_fabsf(hin) * __builtin_amdgcn_exp2f(al * sp);
            if (Av > 0.0f || !(g <= kNegligible))
                atomicOr(&a.flags[(b * (C - 1) + (c - 1)) * (D / 64) + d / 64], 1);
        }
        if (v && c == C - 1 && h_last) h_last[b * DN + dn] = hend;
        carry = __shfl(hend, S - 1, S);
    }
}

// Segment width: the chunk count rounded up to a power of two, at most a wave
int seg_width(int64_t n) {
    int S = 1;
    while (S < n && S < 64) S *= 2;
    return S;
}

template <typename K>
hipError_t launch_seg(K kernels[7], int S, int64_t items, hipStream_t s, const ScanArgs &a) {
    int lg = 0;
    while ((1 << lg) < S) ++lg;
    const int64_t threads = items * S;
    hipLaunchKernelGGL(kernels[lg], dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s, a);
    return launch_status(s);
}

hipError_t launch_combine(const ScanArgs &a, hipStream_t s) {
    void (*k[7])(ScanArgs) = {combine_kernel<1>, combine_kernel<2>, combine_kernel<4>, combine_kernel<8>,
                              combine_kernel<16>, combine_kernel<32>, combine_kernel<64>};
    return launch_seg(k, seg_width(a.n_chunks - 1), a.B * a.D * a.N, s, a);
}

hipError_t launch_local_combine(const ScanArgs &a, float *h_last, hipStream_t s) {
    void (*k[7])(ScanArgs, float *) = {local_combine_kernel<1>, local_combine_kernel<2>, local_combine_kernel<4>,
                                       local_combine_kernel<8>, local_combine_kernel<16>,
                                       local_combine_kernel<32>, local_combine_kernel<64>};
    const int S = seg_width(a.n_chunks);
    int lg = 0;
    while ((1 << lg) < S) ++lg;
    const int64_t threads = a.B * a.D * a.N * S;
    hipLaunchKernelGGL(k[lg], dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s, a, h_last);
    return launch_status(s);
}

// n 16-bit words of zeros (any output of a gradient that has no terms)
__global__ void __launch_bounds__(256) zero16_kernel(uint16_t *p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// h_last = h0 (or zeros) for an empty sequence.
__global__ void __launch_bounds__(256) fill_state_kernel(float *h_last, const float *h0, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) h_last[i] = h0 ? h0[i] : 0.0f;
}


int hip_fail(const char *what, hipError_t e) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return SSM_EHIP;
}

hipError_t launch_scan_any(const ScanArgs &a, dim3 grid, const ScanPlan &p, int disc, bool bf16,
                           bool has_z, bool carry, hipStream_t s) {
    if (p.fast) {
        if (disc == kZOH) return launch_scan_fast_zoh(a, grid, p, bf16, has_z, carry, s);
        if (disc == kBilinear) return launch_scan_fast_bilinear(a, grid, p, bf16, has_z, carry, s);
        return launch_scan_fast_mamba(a, grid, p, bf16, has_z, carry, s);
    }
    if (disc == kZOH) return launch_scan_generic_zoh(a, grid, p, bf16, has_z, carry, s);
    if (disc == kBilinear) return launch_scan_generic_bilinear(a, grid, p, bf16, has_z, carry, s);
    return launch_scan_generic_mamba(a, grid, p, bf16, has_z, carry, s);
}

}  // namespace
}  // namespace ssm

namespace ssm {
namespace {

// The forward on a checked plan: B/C pre-pass, chunk carries and their combine (several
// chunks), then every chunk from its carried-in state producing y (and, given ckpt, the
// state before every 8th step, for the backward).
int run_scan(const ScanPlan &p, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
             const void *x, const void *delta, const float *A, const void *B, const void *C,
             const float *Dskip, const void *z, const float *h0, float *h_last, void *y,
             int delta_softplus, const ssm_variant *variant, void *workspace, float *ckpt,
             int64_t ck_nblk, hipStream_t s) {
    ScanArgs a;
    a.B = batch; a.L = seqlen; a.D = dim; a.N = dstate;
    a.x = x; a.delta = delta; a.z = z; a.Bm = B; a.Cm = C;
    a.A = A; a.Dskip = Dskip; a.h0 = h0; a.h_last = h_last; a.y = y;
    a.softplus = delta_softplus;
    a.dbias = variant_bias(variant);
    const int disc = variant_disc(variant);
    log_call("scan B=%lld L=%lld D=%lld N=%lld dtype=%d disc=%d: %s kernel, %d states/lane, %d waves, %d-step "
             "blocks, %lld chunk(s) of %lld%s, structured-A check %s, workspace %zu B%s",
             (long long)batch, (long long)seqlen, (long long)dim, (long long)dstate, dtype, disc,
             p.fast ? "specialised" : "generic", p.G, p.NW, p.TB, (long long)p.n_chunks, (long long)p.chunk_len,
             p.local && disc != kBilinear && !ckpt ? " (local scans)" : "", p.structured ? "on" : "off",
             p.ws_bytes, ckpt ? ", storing checkpoints" : "");
    a.structured = p.structured ? 1 : 0;
    a.NW = p.NW;
    a.chunk_len = p.chunk_len;
    a.n_chunks = p.n_chunks;
    a.ws_P = p.n_chunks > 1 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + p.ws_P_off) : nullptr;
    a.ws_H = p.n_chunks > 1 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + p.ws_H_off) : nullptr;
    a.ws_BC = p.fast ? reinterpret_cast<float *>(static_cast<char *>(workspace) + p.ws_BC_off) : nullptr;
    a.bc_lpad = p.bc_lpad;
    const unsigned dblocks = static_cast<unsigned>((dim + kChannelsPerBlock - 1) / kChannelsPerBlock);
    const bool bf16 = dtype == SSM_DTYPE_BF16;
    const bool has_z = z != nullptr;
    hipError_t e;
    if (p.fast) {
        // 0) B/C rows of every chunk to fp32, interleaved per state group, zero-padded
        e = launch_bc_pack(a, p, disc, bf16, s);
        if (e != hipSuccess) return hip_fail("B/C pack launch", e);
    }
    if (p.local && disc != kBilinear && !ckpt) {
        // Long chunks, exponential decays: every chunk scanned once from its own start
        // (chunk 0 from h0), its y written except for the first kLocalPrefix steps of chunks
        // >= 1; the carries folded by a parallel scan; those prefixes rescanned from the
        // carried-in states; the rest of a chunk rescanned only where the carried-in state
        // has not died out by then (flags).  About 1.06x the work of one pass, against 1.8x
        // for a carry pass followed by a full rescan.
        const unsigned C = static_cast<unsigned>(p.n_chunks);
        char *wsb = static_cast<char *>(workspace);
        a.ws_Hl = reinterpret_cast<float *>(wsb + p.ws_Hl_off);
        a.S_part = reinterpret_cast<float *>(wsb + p.ws_S_off);
        a.flags = reinterpret_cast<int *>(wsb + p.ws_F_off);
        a.y_skip = kLocalPrefix;
        a.h_last = nullptr;
        e = launch_scan_any(a, dim3(dblocks, static_cast<unsigned>(batch), C), p, disc, bf16, has_z, false, s);
        if (e != hipSuccess) return hip_fail("local scan launch", e);
        e = launch_local_combine(a, h_last, s);
        if (e != hipSuccess) return hip_fail("local carry combine launch", e);
        ScanArgs r = a;   // the prefixes of chunks >= 1, from their carried-in states
        r.ws_Hl = nullptr; r.S_part = nullptr; r.flags = nullptr; r.y_skip = 0;
        r.c_first = 1;
        r.t_span = kLocalPrefix;
        r.h_in = a.ws_H;
        r.h_out = a.ws_P;
        dim3 gr(dblocks, static_cast<unsigned>(batch), C - 1);
        e = launch_scan_any(r, gr, p, disc, bf16, has_z, false, s);
        if (e != hipSuccess) return hip_fail("prefix rescan launch", e);
        r.t_off = kLocalPrefix;   // the rest of the flagged chunks, from the prefix's end state
        r.t_span = 0;
        r.h_in = a.ws_P;
        r.h_out = nullptr;
        r.flag_in = a.flags;
        e = launch_scan_any(r, gr, p, disc, bf16, has_z, false, s);
        if (e != hipSuccess) return hip_fail("continuation rescan launch", e);
        return SSM_OK;
    }
    if (p.n_chunks > 1) {
        // 1) carries of every chunk but the last
        dim3 g1(dblocks, static_cast<unsigned>(batch), static_cast<unsigned>(p.n_chunks - 1));
        e = launch_scan_any(a, g1, p, disc, bf16, false, true, s);
        if (e != hipSuccess) return hip_fail("scan carry launch", e);
        // 2) fold the carries in order
        e = launch_combine(a, s);
        if (e != hipSuccess) return hip_fail("carry combine launch", e);
    }
    // 3) every chunk from its carried-in state, producing y (and the checkpoints)
    dim3 g3(dblocks, static_cast<unsigned>(batch), static_cast<unsigned>(p.n_chunks));
    a.ckpt = ckpt;
    a.ck_nblk = ck_nblk;
    e = ckpt ? launch_scan_save(a, g3, p, disc, bf16, has_z, s) : launch_scan_any(a, g3, p, disc, bf16, has_z, false, s);
    if (e != hipSuccess) return hip_fail("scan launch", e);
    return SSM_OK;
}

}  // namespace
}  // namespace ssm

extern "C" int ssm_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                            const void *x, const void *delta, const float *A, const void *B,
                            const void *C, const float *Dskip, const void *z, const float *h0,
                            float *h_last, void *y, int delta_softplus, const ssm_variant *variant,
                            const ssm_scan_opts *opts, void *workspace, size_t workspace_bytes,
                            void *stream) {
    using namespace ssm;
    clear_error();
    ScanPlan p;
    int st = check_scan(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, h_last,
                        y, delta_softplus, variant, opts, workspace, workspace_bytes, &p);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (seqlen == 0) {
        if (!h_last) return SSM_OK;
        const int64_t n = batch * dim * dstate;
        hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                           0, s, h_last, h0, n);
        hipError_t e = launch_status(s);
        return e == hipSuccess ? SSM_OK : hip_fail("fill_state launch", e);
    }
    return run_scan(p, batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, h_last, y,
                    delta_softplus, variant, workspace, nullptr, 0, s);
}

// ---- the forward for callers that cannot allocate: its workspace is a fixed device array

namespace ssm {
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;   // SSM_NOALLOC_SCRATCH_BYTES
constexpr int kMaxDevices = 64;
// One copy per GPU, held from the library's load until the process ends.  In host code this
// name is not a device address: host code uses the per-device address from
// hipGetSymbolAddress (scratch_ptr) wherever it needs the array's memory.
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the current device (looked up once per device).
int scratch_ptr(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev < 0 || dev >= kMaxDevices) {
        set_error("device %d is beyond the %d devices the fixed scratch supports", dev, kMaxDevices);
        return SSM_EUNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", e);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SSM_OK;
}
}  // namespace
}  // namespace ssm

extern "C" size_t ssm_noalloc_scratch_bytes(void) { return ssm::kScratchBytes; }

extern "C" int ssm_scan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                                    const void *x, const void *delta, const float *A, const void *B,
                                    const void *C, const float *Dskip, const void *z, const float *h0,
                                    float *h_last, void *y, int delta_softplus, const ssm_variant *variant,
                                    const ssm_scan_opts *opts, void *stream) {
    using namespace ssm;
    clear_error();
    ScanPlan p;
    int st = plan_scan(batch, seqlen, dim, dstate, dtype, opts, &p);
    if (st != SSM_OK) return st;
    if (p.ws_bytes > kScratchBytes) {
        set_error("this shape needs %zu bytes of workspace; the fixed scratch holds %zu (use ssm_scan_fwd "
                  "with a caller-allocated workspace)", p.ws_bytes, kScratchBytes);
        return SSM_EWORKSPACE;
    }
    void *ws = nullptr;
    if (p.ws_bytes > 0 && batch > 0 && dim > 0 && seqlen > 0) {
        st = scratch_ptr(&ws);
        if (st != SSM_OK) return st;
    }
    st = check_scan(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, h_last, y,
                    delta_softplus, variant, opts, ws, ws ? kScratchBytes : 0, &p);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (seqlen == 0) {
        if (!h_last) return SSM_OK;
        const int64_t n = batch * dim * dstate;
        hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                           0, s, h_last, h0, n);
        hipError_t e = launch_status(s);
        return e == hipSuccess ? SSM_OK : hip_fail("fill_state launch", e);
    }
    return run_scan(p, batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, h_last, y,
                    delta_softplus, variant, ws, nullptr, 0, s);
}

extern "C" int ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, int dtype, float *h,
                                const void *x, const void *delta, const float *A, const void *B,
                                const void *C, const float *Dskip, const void *z, void *y,
                                int delta_softplus, const ssm_variant *variant, void *stream) {
    using namespace ssm;
    clear_error();
    int st = check_state_update(batch, dim, dstate, dtype, h, x, delta, A, B, C, Dskip, z, y,
                                delta_softplus, variant);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    UpdArgs a;
    a.B = batch; a.D = dim; a.N = dstate; a.h = h;
    a.x = x; a.delta = delta; a.z = z; a.Bm = B; a.Cm = C; a.A = A; a.Dskip = Dskip; a.y = y;
    a.softplus = delta_softplus;
    a.dbias = variant_bias(variant);
    // four states per lane (one 16-byte access when dstate % 4 == 0), one when fewer than 64
    // states are not a multiple of four; at most 64 lanes per channel
    const int G = (dstate % 4 == 0 || dstate > 64) ? 4 : 1;
    int lpc = 1;
    while (lpc * G < dstate) lpc *= 2;
    a.lpc = lpc;
    log_call("state_update B=%lld D=%lld N=%lld dtype=%d: %d states per lane, %d lanes per channel",
             (long long)batch, (long long)dim, (long long)dstate, dtype, G, lpc);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_state_update(a, variant_disc(variant), dtype == SSM_DTYPE_BF16, z != nullptr, s);
    return e == hipSuccess ? SSM_OK : hip_fail("state update launch", e);
}

extern "C" int ssm_scan_fwd_save(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                                 const void *x, const void *delta, const float *A, const void *B,
                                 const void *C, const float *Dskip, const void *z, const float *h0,
                                 float *h_last, void *y, int delta_softplus, const ssm_variant *variant,
                                 float *checkpoints, void *workspace, size_t workspace_bytes, void *stream) {
    using namespace ssm;
    clear_error();
    BwdPlan bp;
    int st = check_scan_save(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, h_last, y,
                             delta_softplus, variant, checkpoints, workspace, workspace_bytes, &bp);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (seqlen == 0) {   // no steps and no checkpoints: h_last = h0
        if (!h_last) return SSM_OK;
        const int64_t n = batch * dim * dstate;
        hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                           0, s, h_last, h0, n);
        hipError_t e = launch_status(s);
        return e == hipSuccess ? SSM_OK : hip_fail("fill_state launch", e);
    }
    return run_scan(bp.fwd, batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, h_last, y,
                    delta_softplus, variant, workspace, checkpoints, bp.nblk, s);
}

namespace ssm {
namespace {

// The backward on the native shape (dstate 16, dim a multiple of 64), after the checks.
int bwd_native(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
               const void *x, const void *delta, const float *A, const void *B,
               const void *C, const float *Dskip, const void *z, const float *h0,
               const void *dy, const float *dh_last, void *dx, void *ddelta, float *dA,
               void *dB, void *dC, float *dD, void *dz, float *dh0, int delta_softplus,
               int discretization, const float *delta_bias, float *ddelta_bias,
               const float *checkpoints, void *workspace, const BwdPlan &p, hipStream_t s,
               int accum = 0) {
    hipError_t e;
    char *ws = static_cast<char *>(workspace);
    const bool bf16 = dtype == SSM_DTYPE_BF16;
    // 1) checkpoints: the specialised forward kernel over the sequence, storing the state
    //    before every 8th step (B/C packed first, as for the forward); with several chunks
    //    the forward's carries and combine come first, and every chunk starts from its
    //    carried-in state.  Skipped when the caller passes the checkpoints that
    //    ssm_scan_fwd_save stored.
    if (!checkpoints) {
        char *fws = ws + p.fwd_off;
        ScanArgs fa;
        fa.B = batch; fa.L = seqlen; fa.D = dim; fa.N = dstate;
        fa.x = x; fa.delta = delta; fa.z = nullptr; fa.Bm = B; fa.Cm = C;
        fa.A = A; fa.Dskip = nullptr; fa.h0 = h0; fa.h_last = nullptr; fa.y = nullptr;
        fa.softplus = delta_softplus;
        fa.dbias = delta_bias;
        fa.structured = p.fwd.structured ? 1 : 0;
        fa.NW = p.fwd.NW;
        fa.chunk_len = p.fwd.chunk_len;
        fa.n_chunks = p.fwd.n_chunks;
        fa.ws_P = p.fwd.n_chunks > 1 ? reinterpret_cast<float *>(fws + p.fwd.ws_P_off) : nullptr;
        fa.ws_H = p.fwd.n_chunks > 1 ? reinterpret_cast<float *>(fws + p.fwd.ws_H_off) : nullptr;
        fa.ws_BC = reinterpret_cast<float *>(fws + p.fwd.ws_BC_off);
        fa.bc_lpad = p.fwd.bc_lpad;
        fa.ckpt = reinterpret_cast<float *>(ws + p.ckpt_off);
        fa.ck_nblk = p.nblk;
        e = launch_bc_pack(fa, p.fwd, discretization, bf16, s);
        if (e != hipSuccess) return hip_fail("B/C pack launch", e);
        const unsigned dblocks = static_cast<unsigned>(dim / 64);
        if (p.fwd.n_chunks > 1) {
            dim3 g1(dblocks, static_cast<unsigned>(batch), static_cast<unsigned>(p.fwd.n_chunks - 1));
            e = launch_scan_any(fa, g1, p.fwd, discretization, bf16, false, true, s);
            if (e != hipSuccess) return hip_fail("checkpoint carry launch", e);
            e = launch_combine(fa, s);
            if (e != hipSuccess) return hip_fail("checkpoint carry combine launch", e);
        }
        e = launch_scan_ckpt(fa, dim3(dblocks, static_cast<unsigned>(batch), static_cast<unsigned>(p.fwd.n_chunks)),
                             p.fwd, discretization, bf16, s);
        if (e != hipSuccess) return hip_fail("checkpoint pass launch", e);
    }
    // 2) the adjoint carries (several chunks), the reverse sweep and the reductions
    BwdArgs a;
    a.B = batch; a.L = seqlen; a.D = dim;
    a.x = x; a.delta = delta; a.z = z; a.dy = dy; a.Bm = B; a.Cm = C;
    a.A = A; a.Dskip = Dskip; a.h0 = h0; a.dh_last = dh_last;
    a.dx = dx; a.ddelta = ddelta; a.dz = dz; a.dB = dB; a.dC = dC;
    a.dA = dA; a.dD = Dskip ? dD : nullptr; a.dh0 = dh0;
    a.softplus = delta_softplus;
    a.nblk = p.nblk;
    a.n_chunks = p.n_chunks;
    a.chunk_len = p.chunk_len;
    a.ckpt = checkpoints ? const_cast<float *>(checkpoints) : reinterpret_cast<float *>(ws + p.ckpt_off);
    a.partBC = reinterpret_cast<float *>(ws + p.partBC_off);
    a.partA = reinterpret_cast<float *>(ws + p.partA_off);
    a.partD = reinterpret_cast<float *>(ws + p.partD_off);
    a.dbias = delta_bias;
    a.ddbias = delta_bias ? ddelta_bias : nullptr;
    a.partDB = reinterpret_cast<float *>(ws + p.partDB_off);
    a.lc_P = p.n_chunks > 1 ? reinterpret_cast<float *>(ws + p.lcP_off) : nullptr;
    a.lc_H = p.n_chunks > 1 ? reinterpret_cast<float *>(ws + p.lcH_off) : nullptr;
    a.accum = accum;
    e = launch_scan_bwd(a, discretization, bf16, z != nullptr, s);
    return e == hipSuccess ? SSM_OK : hip_fail("scan backward launch", e);
}

// dst [n0][m1][m2] from src [n0][n1][n2] (n1 <= m1, n2 <= m2); entries src does not cover
// (or all, when src is null) take fill
template <typename E>
__global__ void __launch_bounds__(256) pad3_kernel(E *dst, const E *src, int64_t n0, int64_t n1, int64_t n2,
                                                   int64_t m1, int64_t m2, E fill) {
    const int64_t total = n0 * m1 * m2;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t i2 = i % m2, r = i / m2, i1 = r % m1, i0 = r / m1;
        dst[i] = (src && i1 < n1 && i2 < n2) ? src[(i0 * n1 + i1) * n2 + i2] : fill;
    }
}

// dst [n0][n1][n2] from the leading block of src [n0][m1][m2]
template <typename E>
__global__ void __launch_bounds__(256) unpad3_kernel(E *dst, const E *src, int64_t n0, int64_t n1, int64_t n2,
                                                     int64_t m1, int64_t m2) {
    const int64_t total = n0 * n1 * n2;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t i2 = i % n2, r = i / n2, i1 = r % n1, i0 = r / n1;
        dst[i] = src[(i0 * m1 + i1) * m2 + i2];
    }
}

dim3 grid_for(int64_t n) {
    const int64_t b = (n + 255) / 256;
    return dim3(static_cast<unsigned>(b < 1 ? 1 : b > 16384 ? 16384 : b));
}

// es-byte elements (2 or 4); fill as a float (its bf16 bits for 2-byte elements)
hipError_t pad3(void *dst, const void *src, int64_t n0, int64_t n1, int64_t n2, int64_t m1, int64_t m2,
                size_t es, float fill, hipStream_t s) {
    const dim3 g = grid_for(n0 * m1 * m2);
    if (es == 2)
        hipLaunchKernelGGL(pad3_kernel<uint16_t>, g, dim3(256), 0, s, static_cast<uint16_t *>(dst),
                           static_cast<const uint16_t *>(src), n0, n1, n2, m1, m2,
                           static_cast<uint16_t>(__builtin_bit_cast(uint32_t, fill) >> 16));
    else
        hipLaunchKernelGGL(pad3_kernel<float>, g, dim3(256), 0, s, static_cast<float *>(dst),
                           static_cast<const float *>(src), n0, n1, n2, m1, m2, fill);
    return launch_status(s);
}

hipError_t unpad3(void *dst, const void *src, int64_t n0, int64_t n1, int64_t n2, int64_t m1, int64_t m2,
                  size_t es, hipStream_t s) {
    const dim3 g = grid_for(n0 * n1 * n2);
    if (es == 2)
        hipLaunchKernelGGL(unpad3_kernel<uint16_t>, g, dim3(256), 0, s, static_cast<uint16_t *>(dst),
                           static_cast<const uint16_t *>(src), n0, n1, n2, m1, m2);
    else
        hipLaunchKernelGGL(unpad3_kernel<float>, g, dim3(256), 0, s, static_cast<float *>(dst),
                           static_cast<const float *>(src), n0, n1, n2, m1, m2);
    return launch_status(s);
}

// dst [n0][m1][m2] (Eo) from columns c0 .. c0 + m2 - 1 of src [n0][n1][n2] (Ei), converted;
// rows past n1, columns past n2 and an absent src take fill
template <typename Eo, typename Ei>
__global__ void __launch_bounds__(256) gpad3_kernel(Eo *dst, const Ei *src, int64_t n0, int64_t n1, int64_t n2,
                                                    int64_t c0, int64_t m1, int64_t m2, float fill) {
    const int64_t total = n0 * m1 * m2;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t i2 = i % m2, r = i / m2, i1 = r % m1, i0 = r / m1, c = c0 + i2;
        put(dst, i, (src && i1 < n1 && c < n2) ? widen(src, (i0 * n1 + i1) * n2 + c) : fill);
    }
}

// columns c0 .. c0 + w - 1 of dst [n0][n1][n2] (Eo) from the leading w columns of
// src [n0][n1][m2] (Ei), converted (w = min(m2, n2 - c0))
template <typename Eo, typename Ei>
__global__ void __launch_bounds__(256) gunpad3_kernel(Eo *dst, const Ei *src, int64_t n0, int64_t n1, int64_t n2,
                                                      int64_t c0, int64_t m1, int64_t m2, int64_t w) {
    const int64_t total = n0 * n1 * w;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t i2 = i % w, r = i / w, i1 = r % n1, i0 = r / n1;
        put(dst, (i0 * n1 + i1) * n2 + c0 + i2, widen(src, (i0 * m1 + i1) * m2 + i2));
    }
}

// dst[i] = src[i] converted, i < n: the copies above when they are flat (no padding, no
// column offset), without their index arithmetic
template <typename Eo, typename Ei>
__global__ void __launch_bounds__(256) convert_kernel(Eo *dst, const Ei *src, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * 256)
        put(dst, i, widen(src, i));
}

__global__ void __launch_bounds__(256) add_kernel(float *dst, const float *src, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * 256)
        dst[i] += src[i];
}

// es-byte elements in and out (2: bf16, 4: fp32)
hipError_t gpad3(void *dst, size_t eo, const void *src, size_t ei, int64_t n0, int64_t n1, int64_t n2, int64_t c0,
                 int64_t m1, int64_t m2, float fill, hipStream_t s) {
    const dim3 g = grid_for(n0 * m1 * m2);
    if (src && n1 == 1 && m1 == 1 && c0 == 0 && m2 == n2 && eo == 4) {
        if (ei == 2)
            hipLaunchKernelGGL((convert_kernel<float, uint16_t>), g, dim3(256), 0, s, static_cast<float *>(dst),
                               static_cast<const uint16_t *>(src), n0 * n2);
        else if (ei == 4)
            hipLaunchKernelGGL((convert_kernel<float, float>), g, dim3(256), 0, s, static_cast<float *>(dst),
                               static_cast<const float *>(src), n0 * n2);
        else
            return hipErrorInvalidValue;
        return launch_status(s);
    }
    if (eo == 4 && ei == 2)
        hipLaunchKernelGGL((gpad3_kernel<float, uint16_t>), g, dim3(256), 0, s, static_cast<float *>(dst),
                           static_cast<const uint16_t *>(src), n0, n1, n2, c0, m1, m2, fill);
    else if (eo == 4 && ei == 4)
        hipLaunchKernelGGL((gpad3_kernel<float, float>), g, dim3(256), 0, s, static_cast<float *>(dst),
                           static_cast<const float *>(src), n0, n1, n2, c0, m1, m2, fill);
    else
        return hipErrorInvalidValue;
    return launch_status(s);
}

hipError_t gunpad3(void *dst, size_t eo, const void *src, size_t ei, int64_t n0, int64_t n1, int64_t n2, int64_t c0,
                   int64_t m1, int64_t m2, hipStream_t s) {
    const int64_t w = m2 < n2 - c0 ? m2 : n2 - c0;
    if (w <= 0) return hipSuccess;
    const dim3 g = grid_for(n0 * n1 * w);
    if (n1 == 1 && m1 == 1 && c0 == 0 && m2 == n2 && ei == 4) {
        if (eo == 2)
            hipLaunchKernelGGL((convert_kernel<uint16_t, float>), g, dim3(256), 0, s, static_cast<uint16_t *>(dst),
                               static_cast<const float *>(src), n0 * n2);
        else if (eo == 4)
            hipLaunchKernelGGL((convert_kernel<float, float>), g, dim3(256), 0, s, static_cast<float *>(dst),
                               static_cast<const float *>(src), n0 * n2);
        else
            return hipErrorInvalidValue;
        return launch_status(s);
    }
    if (eo == 2 && ei == 4)
        hipLaunchKernelGGL((gunpad3_kernel<uint16_t, float>), g, dim3(256), 0, s, static_cast<uint16_t *>(dst),
                           static_cast<const float *>(src), n0, n1, n2, c0, m1, m2, w);
    else if (eo == 4 && ei == 4)
        hipLaunchKernelGGL((gunpad3_kernel<float, float>), g, dim3(256), 0, s, static_cast<float *>(dst),
                           static_cast<const float *>(src), n0, n1, n2, c0, m1, m2, w);
    else
        return hipErrorInvalidValue;
    return launch_status(s);
}

// dst[i] = src[i / R] (converted to fp32), i < n * R
template <typename Ei>
__global__ void __launch_bounds__(256) repeat_kernel(float *dst, const Ei *src, int64_t n, int64_t R) {
    const int64_t total = n * R;
    if (total <= 0x7fffffff) {   // 32-bit index arithmetic where it fits
        const uint32_t t32 = static_cast<uint32_t>(total), r32 = static_cast<uint32_t>(R);
        for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < t32; i += gridDim.x * 256u)
            dst[i] = widen(src, i / r32);
        return;
    }
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * 256)
        dst[i] = widen(src, i / R);
}

// dst[i] = sum of src[i * S .. i * S + S - 1] (converted to Eo), i < n: one wavefront per
// output (i is wave-uniform), lane j adding elements j, j + 64, ... in order, then a fixed
// butterfly over the lanes, lane 0's result stored (the same order on every call)
template <typename Eo>
__global__ void __launch_bounds__(256) segsum_kernel(Eo *dst, const float *src, int64_t n, int64_t S) {
    const int lane = threadIdx.x & 63;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); i < n;
         i += static_cast<int64_t>(gridDim.x) * 4) {
        float acc = 0.0f;
        for (int64_t j = lane; j < S; j += 64) acc += src[i * S + j];
        for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
        if (lane == 0) put(dst, i, acc);
    }
}

hipError_t repeat_f32(float *dst, const void *src, size_t ei, int64_t n, int64_t R, hipStream_t s) {
    const dim3 g = grid_for(n * R);
    if (ei == 2)
        hipLaunchKernelGGL(repeat_kernel<uint16_t>, g, dim3(256), 0, s, dst, static_cast<const uint16_t *>(src), n, R);
    else
        hipLaunchKernelGGL(repeat_kernel<float>, g, dim3(256), 0, s, dst, static_cast<const float *>(src), n, R);
    return launch_status(s);
}

hipError_t segsum(void *dst, size_t eo, const float *src, int64_t n, int64_t S, hipStream_t s) {
    const dim3 g = grid_for(n * 64);   // four outputs per 256-thread block
    if (eo == 2)
        hipLaunchKernelGGL(segsum_kernel<uint16_t>, g, dim3(256), 0, s, static_cast<uint16_t *>(dst), src, n, S);
    else
        hipLaunchKernelGGL(segsum_kernel<float>, g, dim3(256), 0, s, static_cast<float *>(dst), src, n, S);
    return launch_status(s);
}

hipError_t add_f32(float *dst, const float *src, int64_t n, hipStream_t s) {
    hipLaunchKernelGGL(add_kernel, grid_for(n), dim3(256), 0, s, dst, src, n);
    return launch_status(s);
}

}  // namespace
}  // namespace ssm

extern "C" int ssm_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                            const void *x, const void *delta, const float *A, const void *B,
                            const void *C, const float *Dskip, const void *z, const float *h0,
                            const void *dy, const float *dh_last, void *dx, void *ddelta, float *dA,
                            void *dB, void *dC, float *dD, void *dz, float *dh0, int delta_softplus,
                            int discretization, const float *delta_bias, float *ddelta_bias,
                            const float *checkpoints, void *workspace, size_t workspace_bytes,
                            void *stream) {
    using namespace ssm;
    clear_error();
    BwdPlan p;
    int st = check_scan_bwd(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, dy,
                            dh_last, dx, ddelta, dA, dB, dC, dD, dz, dh0, delta_softplus, discretization,
                            delta_bias, ddelta_bias, checkpoints, workspace, workspace_bytes, &p);
    if (st != SSM_OK) return st;
    log_call("scan_bwd B=%lld L=%lld D=%lld N=%lld dtype=%d disc=%d: %s, %lld chunk(s) of %lld, %s, workspace %zu B",
             (long long)batch, (long long)seqlen, (long long)dim, (long long)dstate, dtype, discretization,
             p.pad ? (p.K > 1 ? "native kernels per group of 16 states on fp32 copies" : "native kernels on padded copies")
                   : "native kernels", (long long)p.n_chunks,
             (long long)p.chunk_len, checkpoints ? "saved checkpoints" : "own checkpoint pass",
             checkpoints ? p.ws_bytes_saved : p.ws_bytes);
    if (dim == 0) return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (batch == 0 || seqlen == 0) {
        // no rows or no steps: dh0 = dh_last, and the reductions over rows and steps are zero
        if (dh0 && batch > 0) {
            const int64_t n = batch * dim * dstate;
            hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                               0, s, dh0, dh_last, n);
            e = launch_status(s);
            if (e != hipSuccess) return hip_fail("fill_state launch", e);
        }
        hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((dim * dstate + 255) / 256)),
                           dim3(256), 0, s, dA, static_cast<const float *>(nullptr), dim * dstate);
        e = launch_status(s);
        if (e != hipSuccess) return hip_fail("fill_state launch", e);
        if (Dskip && dD) {
            hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((dim + 255) / 256)), dim3(256),
                               0, s, dD, static_cast<const float *>(nullptr), dim);
            e = launch_status(s);
            if (e != hipSuccess) return hip_fail("fill_state launch", e);
        }
        if (delta_bias) {
            hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((dim + 255) / 256)), dim3(256),
                               0, s, ddelta_bias, static_cast<const float *>(nullptr), dim);
            e = launch_status(s);
            if (e != hipSuccess) return hip_fail("fill_state launch", e);
        }
        return SSM_OK;
    }
    char *ws = static_cast<char *>(workspace);
    if (p.pad && p.K > 1) {
        // more than 16 states: the native backward once per group of 16 states, on fp32
        // copies; the states of one group neither read nor write another's, and the
        // per-channel gradients are linear in the per-state terms, so they are the groups'
        // sums (D and its terms in group 0 only)
        BwdPlan in;
        st = plan_scan_bwd(batch, seqlen, p.Dp, 16, SSM_DTYPE_F32, &in);
        if (st != SSM_OK) return st;
        const size_t es = dtype_size(dtype);
        const int64_t BL = batch * seqlen, Dp = p.Dp, N = dstate;
        auto at = [&](int i) { return static_cast<void *>(ws + p.pad_off[i]); };
        auto atf = [&](int i) { return reinterpret_cast<float *>(ws + p.pad_off[i]); };
        // fp32 tokens that need no padding are read in place, and the per-channel gradients
        // are summed straight into the caller's outputs (which overlap no input)
        const bool direct = p.direct;
        const void *tx = direct ? x : at(kPX), *tdl = direct ? delta : at(kPDelta);
        const void *tz = direct ? z : at(kPZ), *tdy = direct ? dy : at(kPDy);
        struct { void *dst; const void *src; int64_t n0, n1, n2, m1, m2; size_t es; } toks[] = {
            {at(kPX), direct ? nullptr : x, BL, 1, dim, 1, Dp, es},
            {at(kPDelta), direct ? nullptr : delta, BL, 1, dim, 1, Dp, es},
            {at(kPZ), direct ? nullptr : z, BL, 1, dim, 1, Dp, es},
            {at(kPDy), direct ? nullptr : dy, BL, 1, dim, 1, Dp, es},
            {at(kPDskip), Dskip, 1, 1, dim, 1, Dp, 4},
            {at(kPBias), delta_bias, 1, 1, dim, 1, Dp, 4},
        };
        for (const auto &c : toks) {
            if (!c.src) continue;
            e = gpad3(c.dst, 4, c.src, c.es, c.n0, c.n1, c.n2, 0, c.m1, c.m2, 0.0f, s);
            if (e != hipSuccess) return hip_fail("pad launch", e);
        }
        for (int64_t g = 0; g < p.K; ++g) {
            const int64_t c0 = 16 * g;
            struct { void *dst; const void *src; int64_t n0, n1, n2, m1, m2; size_t es; float fill; } ins[] = {
                {at(kPB), B, BL, 1, N, 1, 16, es, 0.0f},
                {at(kPC), C, BL, 1, N, 1, 16, es, 0.0f},
                {at(kPA), A, 1, dim, N, Dp, 16, 4, -1.0f},
                {at(kPH0), h0, batch, dim, N, Dp, 16, 4, 0.0f},
                {at(kPDhLast), dh_last, batch, dim, N, Dp, 16, 4, 0.0f},
            };
            for (const auto &c : ins) {
                if (!c.src && c.dst != at(kPA)) continue;
                e = gpad3(c.dst, 4, c.src, c.es, c.n0, c.n1, c.n2, c0, c.m1, c.m2, c.fill, s);
                if (e != hipSuccess) return hip_fail("pad launch", e);
            }
            // the per-channel gradients go straight into their sums: group 0 stores them, the
            // later groups' kernels add theirs to what the sums hold; the bias's gradient (a
            // reduction over rows and steps) is added after each later group
            const bool g0 = g == 0;
            float *gdx = direct ? static_cast<float *>(dx) : atf(kSDx);
            float *gdd = direct ? static_cast<float *>(ddelta) : atf(kSDdelta);
            float *gdz = direct ? static_cast<float *>(dz) : atf(kSDz);
            float *gdb = g0 ? atf(kSDBias) : atf(kPDBias);
            st = bwd_native(batch, seqlen, Dp, 16, SSM_DTYPE_F32, tx, tdl, atf(kPA), at(kPB), at(kPC),
                            (g0 && Dskip) ? atf(kPDskip) : nullptr, z ? tz : nullptr,
                            h0 ? atf(kPH0) : nullptr, tdy, dh_last ? atf(kPDhLast) : nullptr, gdx, gdd,
                            atf(kPDA), at(kPDB), at(kPDC), (g0 && Dskip) ? atf(kPDD) : nullptr,
                            z ? static_cast<void *>(gdz) : nullptr, dh0 ? atf(kPDh0) : nullptr, delta_softplus,
                            discretization, delta_bias ? atf(kPBias) : nullptr, delta_bias ? gdb : nullptr,
                            nullptr, ws + p.inner_off, in, s, g0 ? 0 : 1);
            if (st != SSM_OK) return st;
            if (!g0 && delta_bias) {
                e = add_f32(atf(kSDBias), gdb, Dp, s);
                if (e != hipSuccess) return hip_fail("sum launch", e);
            }
            // this group's columns of the per-state gradients
            struct { void *dst; const void *src; int64_t n0, n1, n2, m1, m2; size_t es; } outs[] = {
                {dB, at(kPDB), BL, 1, N, 1, 16, es},
                {dC, at(kPDC), BL, 1, N, 1, 16, es},
                {dA, at(kPDA), 1, dim, N, Dp, 16, 4},
                {dh0, at(kPDh0), batch, dim, N, Dp, 16, 4},
            };
            for (const auto &c : outs) {
                if (!c.dst) continue;
                e = gunpad3(c.dst, c.es, c.src, 4, c.n0, c.n1, c.n2, c0, c.m1, c.m2, s);
                if (e != hipSuccess) return hip_fail("unpad launch", e);
            }
        }
        struct { void *dst; const void *src; int64_t n0, n1, n2, m1, m2; size_t es; } outs[] = {
            {direct ? nullptr : dx, at(kSDx), BL, 1, dim, 1, Dp, es},
            {direct ? nullptr : ddelta, at(kSDdelta), BL, 1, dim, 1, Dp, es},
            {(z && !direct) ? dz : nullptr, at(kSDz), BL, 1, dim, 1, Dp, es},
            {Dskip ? dD : nullptr, at(kPDD), 1, 1, dim, 1, Dp, 4},
            {delta_bias ? ddelta_bias : nullptr, at(kSDBias), 1, 1, dim, 1, Dp, 4},
        };
        for (const auto &c : outs) {
            if (!c.dst) continue;
            e = gunpad3(c.dst, c.es, c.src, 4, c.n0, c.n1, c.n2, 0, c.m1, c.m2, s);
            if (e != hipSuccess) return hip_fail("unpad launch", e);
        }
        return SSM_OK;
    }
    if (p.pad) {
        // dstate < 16 or dim not a multiple of 64: the native backward on padded copies
        BwdPlan in;
        st = plan_scan_bwd(batch, seqlen, p.Dp, 16, dtype, &in);
        if (st != SSM_OK) return st;
        const size_t es = dtype_size(dtype);
        const int64_t BL = batch * seqlen, Dp = p.Dp, N = dstate;
        auto at = [&](int i) { return static_cast<void *>(ws + p.pad_off[i]); };
        auto atf = [&](int i) { return reinterpret_cast<float *>(ws + p.pad_off[i]); };
        // inputs: tokens [B L D] -> [B L Dp], B/C [B L N] -> [B L 16], A [D N] -> [Dp 16] (-1 outside),
        // D and the bias [D] -> [Dp], h0 and dh_last [B D N] -> [B Dp 16]
        struct { void *dst; const void *src; int64_t n0, n1, n2, m1, m2; size_t es; float fill; } ins[] = {
            {at(kPX), x, BL, 1, dim, 1, Dp, es, 0.0f},
            {at(kPDelta), delta, BL, 1, dim, 1, Dp, es, 0.0f},
            {at(kPZ), z, BL, 1, dim, 1, Dp, es, 0.0f},
            {at(kPDy), dy, BL, 1, dim, 1, Dp, es, 0.0f},
            {at(kPB), B, BL, 1, N, 1, 16, es, 0.0f},
            {at(kPC), C, BL, 1, N, 1, 16, es, 0.0f},
            {at(kPA), A, 1, dim, N, Dp, 16, 4, -1.0f},
            {at(kPDskip), Dskip, 1, 1, dim, 1, Dp, 4, 0.0f},
            {at(kPBias), delta_bias, 1, 1, dim, 1, Dp, 4, 0.0f},
            {at(kPH0), h0, batch, dim, N, Dp, 16, 4, 0.0f},
            {at(kPDhLast), dh_last, batch, dim, N, Dp, 16, 4, 0.0f},
        };
        for (const auto &c : ins) {
            if (!c.src && c.dst != at(kPA)) continue;   // absent optional inputs stay absent
            e = pad3(c.dst, c.src, c.n0, c.n1, c.n2, c.m1, c.m2, c.es, c.fill, s);
            if (e != hipSuccess) return hip_fail("pad launch", e);
        }
        st = bwd_native(batch, seqlen, Dp, 16, dtype, at(kPX), at(kPDelta), atf(kPA), at(kPB), at(kPC),
                        Dskip ? atf(kPDskip) : nullptr, z ? at(kPZ) : nullptr, h0 ? atf(kPH0) : nullptr,
                        at(kPDy), dh_last ? atf(kPDhLast) : nullptr, at(kPDx), at(kPDdelta), atf(kPDA),
                        at(kPDB), at(kPDC), Dskip ? atf(kPDD) : nullptr, z ? at(kPDz) : nullptr,
                        dh0 ? atf(kPDh0) : nullptr, delta_softplus, discretization,
                        delta_bias ? atf(kPBias) : nullptr, delta_bias ? atf(kPDBias) : nullptr, nullptr,
                        ws + p.inner_off, in, s);
        if (st != SSM_OK) return st;
        struct { void *dst; const void *src; int64_t n0, n1, n2, m1, m2; size_t es; } outs[] = {
            {dx, at(kPDx), BL, 1, dim, 1, Dp, es},
            {ddelta, at(kPDdelta), BL, 1, dim, 1, Dp, es},
            {z ? dz : nullptr, at(kPDz), BL, 1, dim, 1, Dp, es},
            {dB, at(kPDB), BL, 1, N, 1, 16, es},
            {dC, at(kPDC), BL, 1, N, 1, 16, es},
            {dA, at(kPDA), 1, dim, N, Dp, 16, 4},
            {Dskip ? dD : nullptr, at(kPDD), 1, 1, dim, 1, Dp, 4},
            {delta_bias ? ddelta_bias : nullptr, at(kPDBias), 1, 1, dim, 1, Dp, 4},
            {dh0, at(kPDh0), batch, dim, N, Dp, 16, 4},
        };
        for (const auto &c : outs) {
            if (!c.dst) continue;
            e = unpad3(c.dst, c.src, c.n0, c.n1, c.n2, c.m1, c.m2, c.es, s);
            if (e != hipSuccess) return hip_fail("unpad launch", e);
        }
        return SSM_OK;
    }
    return bwd_native(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, dy, dh_last, dx,
                      ddelta, dA, dB, dC, dD, dz, dh0, delta_softplus, discretization, delta_bias,
                      ddelta_bias, checkpoints, workspace, p, s);
}

extern "C" int ssm_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int dtype,
                              const void *x, const float *w, const float *bias, const void *state_in,
                              void *y, void *state_out, int silu, void *stream) {
    using namespace ssm;
    clear_error();
    int st = check_conv1d_fwd(batch, seqlen, dim, width, dtype, x, w, bias, state_in, y, state_out, silu);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0 || (seqlen == 0 && (!state_out || width == 1))) return SSM_OK;
    ConvArgs a;
    a.B = batch; a.L = seqlen; a.D = dim; a.W = static_cast<int>(width);
    a.x = x; a.w = w; a.bias = bias; a.state_in = state_in; a.y = y; a.state_out = state_out; a.silu = silu;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // (with seqlen == 0 only the state passes through)
    hipError_t e = launch_conv1d_fwd(a, dtype == SSM_DTYPE_BF16, s);
    return e == hipSuccess ? SSM_OK : hip_fail("conv1d launch", e);
}

extern "C" size_t ssm_conv1d_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                                                 int dtype) {
    (void)dtype;
    return ssm::conv1d_bwd_ws_bytes(batch, seqlen, dim, width);
}

extern "C" int ssm_conv1d_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int dtype,
                              const void *x, const float *w, const float *bias, const void *state_in,
                              const void *dy, void *dx, float *dw, float *dbias, void *dstate, int silu,
                              void *workspace, size_t workspace_bytes, void *stream) {
    using namespace ssm;
    clear_error();
    int st = check_conv1d_bwd(batch, seqlen, dim, width, dtype, x, w, bias, state_in, dy, dx, dw, dbias, dstate,
                              silu, workspace, workspace_bytes);
    if (st != SSM_OK) return st;
    if (dim == 0) return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (width == 1) dstate = nullptr;
    hipError_t e;
    if (batch == 0 || seqlen == 0) {
        // no rows or no steps: every gradient is zero
        auto zero = [&](void *p, int64_t bytes) {
            if (!p || bytes <= 0) return hipSuccess;
            const int64_t n = bytes / 2;
            hipLaunchKernelGGL(zero16_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                               static_cast<uint16_t *>(p), n);
            return launch_status(s);
        };
        e = zero(dw, dim * width * 4);
        if (e == hipSuccess) e = zero(dbias, dim * 4);
        if (e == hipSuccess) e = zero(dstate, batch * dim * (width - 1) * static_cast<int64_t>(dtype_size(dtype)));
        return e == hipSuccess ? SSM_OK : hip_fail("zero fill launch", e);
    }
    ConvArgs a;
    a.B = batch; a.L = seqlen; a.D = dim; a.W = static_cast<int>(width);
    a.x = x; a.w = w; a.bias = bias; a.state_in = state_in; a.y = nullptr; a.state_out = nullptr; a.silu = silu;
    a.dy = dy; a.dx = dx; a.dw = dw; a.dbias = dbias; a.dstate = dstate;
    a.part = static_cast<float *>(workspace);
    e = launch_conv1d_bwd(a, dtype == SSM_DTYPE_BF16, s);
    return e == hipSuccess ? SSM_OK : hip_fail("conv1d backward launch", e);
}

extern "C" int ssm_conv1d_update(int64_t batch, int64_t dim, int64_t width, int dtype, void *state,
                                 const void *x, const float *w, const float *bias, void *y, int silu,
                                 void *stream) {
    using namespace ssm;
    clear_error();
    int st = check_conv1d_update(batch, dim, width, dtype, state, x, w, bias, y, silu);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    ConvArgs a;
    a.B = batch; a.L = 1; a.D = dim; a.W = static_cast<int>(width);
    a.x = x; a.w = w; a.bias = bias; a.state_in = nullptr; a.y = y; a.state_out = state; a.silu = silu;
    hipError_t e = launch_conv1d_update(a, dtype == SSM_DTYPE_BF16, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : hip_fail("conv1d update launch", e);
}

extern "C" int ssm_ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                           int64_t ngroups, int dtype, const void *x, const void *delta, const float *A, const void *B,
                           const void *C, const float *Dskip, const void *z, const float *delta_bias,
                           const float *h0, float *h_last, void *y, int delta_softplus, void *stream) {
    using namespace ssm;
    clear_error();
    int st = check_ssd(batch, seqlen, nheads, headdim, dstate, ngroups, dtype, x, delta, A, B, C, Dskip, z, delta_bias,
                       h0, h_last, y, delta_softplus);
    if (st != SSM_OK) return st;
    if (batch == 0 || nheads == 0) return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (seqlen == 0) {
        if (!h_last) return SSM_OK;
        const int64_t n = batch * nheads * headdim * dstate;
        hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                           h_last, h0, n);
        hipError_t e = launch_status(s);
        return e == hipSuccess ? SSM_OK : hip_fail("fill_state launch", e);
    }
    log_call("ssd B=%lld L=%lld H=%lld P=%lld N=%lld groups=%lld dtype=%d: %s", (long long)batch,
             (long long)seqlen, (long long)nheads, (long long)headdim, (long long)dstate, (long long)ngroups, dtype,
             headdim == 64 && dstate == 128 && dtype == SSM_DTYPE_BF16 ? "matrix-core kernel"
                                                                       : "generic scan kernel, multi-head layout");
    if (headdim != 64 || dstate != 128 || dtype != SSM_DTYPE_BF16) {
        // other head dims, state sizes and fp32: the generic scan kernel over the H * P
        // channels in its multi-head layout (one step size, decay, D and bias per head; B, C
        // shared), in one pass (no workspace)
        const int64_t dim = nheads * headdim;
        ssm_scan_opts o = {seqlen, 0, 8, 0, -1};
        ScanPlan p;
        st = plan_scan(batch, seqlen, dim, dstate, dtype, &o, &p);
        if (st != SSM_OK) return st;
        ScanArgs a;
        a.B = batch; a.L = seqlen; a.D = dim; a.N = dstate;
        a.x = x; a.delta = delta; a.z = z; a.Bm = B; a.Cm = C;
        a.A = A; a.Dskip = Dskip; a.h0 = h0; a.h_last = h_last; a.y = y;
        a.softplus = delta_softplus;
        a.dbias = delta_bias;
        a.NW = p.NW;
        a.chunk_len = p.chunk_len;
        a.n_chunks = 1;
        a.ws_P = a.ws_H = a.ws_BC = nullptr;
        a.bc_lpad = 0;
        a.head_dim = headdim;
        a.bc_groups = ngroups;
        a.bc_group_ch = (nheads / ngroups) * headdim;
        const dim3 g(static_cast<unsigned>((dim + kChannelsPerBlock - 1) / kChannelsPerBlock),
                     static_cast<unsigned>(batch), 1);
        hipError_t e = launch_scan_any(a, g, p, kMamba, dtype == SSM_DTYPE_BF16, z != nullptr, false, s);
        return e == hipSuccess ? SSM_OK : hip_fail("ssd (generic) launch", e);
    }
    SsdArgs a;
    a.B = batch; a.L = seqlen; a.H = nheads; a.G = ngroups;
    a.x = x; a.delta = delta; a.z = z; a.Bm = B; a.Cm = C;
    a.A = A; a.Dskip = Dskip; a.dbias = delta_bias; a.h0 = h0; a.h_last = h_last; a.y = y;
    a.softplus = delta_softplus;
    hipError_t e = launch_ssd(a, s);
    return e == hipSuccess ? SSM_OK : hip_fail("ssd launch", e);
}

namespace ssm {
namespace {
// Workspace of ssm_ssd_bwd: fp32 per-channel copies of the inputs (tokens over the H * P
// channels, each head's step size, decay, D and bias repeated over its channels), the
// per-channel gradients of the scan backward, then that backward's own workspace.
enum SsdBwdBuf { kQX, kQDelta, kQZ, kQDy, kQB, kQC, kQA, kQD, kQBias,
                 kQDx, kQDdelta, kQDz, kQDB, kQDC, kQDA, kQDD, kQDBias, kQInner, kQBufs };

size_t ssd_bwd_layout(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                      size_t off[kQBufs]) {
    const size_t B = static_cast<size_t>(batch), L = static_cast<size_t>(seqlen);
    const size_t Dc = static_cast<size_t>(nheads * headdim), N = static_cast<size_t>(dstate), f = sizeof(float);
    const size_t tok = B * L * Dc * f, bc = B * L * N * f;
    const size_t bytes[kQInner] = {tok, tok, tok, tok, bc, bc, Dc * N * f, Dc * f, Dc * f,
                                   tok, tok, tok, bc, bc, Dc * N * f, Dc * f, Dc * f};
    size_t ws = 0;
    for (int i = 0; i < kQInner; ++i) {
        off[i] = ws;
        ws = (ws + bytes[i] + kWsAlign - 1) / kWsAlign * kWsAlign;
    }
    off[kQInner] = ws;
    return ws + ssm_scan_bwd_workspace_bytes(batch, seqlen, nheads * headdim, dstate, SSM_DTYPE_F32, 0);
}
}  // namespace
}  // namespace ssm

extern "C" size_t ssm_ssd_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                              int64_t dstate, int dtype) {
    using namespace ssm;
    if ((dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16) || batch <= 0 || seqlen <= 0 || nheads <= 0 ||
        headdim < 1 || dstate < 1 || dstate > SSM_MAX_DSTATE)
        return 0;
    size_t off[kQBufs];
    return ssd_bwd_layout(batch, seqlen, nheads, headdim, dstate, off);
}

extern "C" int ssm_ssd_bwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                           int64_t ngroups, int dtype, const void *x, const void *delta, const float *A, const void *B,
                           const void *C, const float *Dskip, const void *z, const float *delta_bias,
                           const float *h0, const void *dy, const float *dh_last, void *dx, void *ddelta, float *dA,
                           void *dB, void *dC, float *dD, void *dz, float *ddelta_bias, float *dh0,
                           int delta_softplus, void *workspace, size_t workspace_bytes, void *stream) {
    using namespace ssm;
    clear_error();
    int st = check_ssd(batch, seqlen, nheads, headdim, dstate, ngroups, dtype, x, delta, A, B, C, Dskip, z,
                       delta_bias, h0, nullptr, dx, delta_softplus);
    if (st != SSM_OK) return st;
    if (ngroups != 1) {
        set_error("ssm_ssd_bwd takes one B/C group (got ngroups=%lld)", (long long)ngroups);
        return SSM_EUNSUPPORTED;
    }
    const bool any = batch > 0 && seqlen > 0 && nheads > 0;
    if (any && (!dy || !dx || !ddelta || !dA || !dB || !dC)) {
        set_error("dy, dx, ddelta, dA, dB and dC are required");
        return SSM_EINVAL;
    }
    if ((Dskip && !dD) || (z && !dz) || (delta_bias && !ddelta_bias)) {
        set_error("dD, dz and ddelta_bias are required with D, z and delta_bias");
        return SSM_EINVAL;
    }
    if (nheads == 0) return SSM_OK;
    size_t off[kQBufs];
    const size_t need = ssd_bwd_layout(batch, seqlen, nheads, headdim, dstate, off);
    if (any && (!workspace || workspace_bytes < need)) {
        set_error("workspace of %zu bytes is too small (need %zu)", workspace_bytes, need);
        return SSM_EWORKSPACE;
    }
    log_call("ssd_bwd B=%lld L=%lld H=%lld P=%lld N=%lld dtype=%d: the scan backward on the %lld channels "
             "(fp32 copies), tied gradients summed per head", (long long)batch, (long long)seqlen,
             (long long)nheads, (long long)headdim, (long long)dstate, dtype, (long long)(nheads * headdim));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t Dc = nheads * headdim, P = headdim, N = dstate, BL = batch * seqlen;
    const size_t es = dtype_size(dtype);
    char *ws = static_cast<char *>(workspace);
    auto q = [&](int i) { return reinterpret_cast<float *>(ws + off[i]); };
    hipError_t e = hipSuccess;
    if (!any) {
        // no rows or no steps: the per-head gradients are zero, dh0 = dh_last (or zeros)
        auto fill = [&](float *d, const float *src, int64_t n) {
            if (!d || n <= 0) return hipSuccess;
            hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, d,
                               src, n);
            return launch_status(s);
        };
        e = fill(dA, nullptr, nheads);
        if (e == hipSuccess && Dskip) e = fill(dD, nullptr, nheads);
        if (e == hipSuccess && delta_bias) e = fill(ddelta_bias, nullptr, nheads);
        if (e == hipSuccess && batch > 0) e = fill(dh0, dh_last, batch * Dc * N);
        return e == hipSuccess ? SSM_OK : hip_fail("fill_state launch", e);
    }
    // the per-channel expansion (fp32): tokens converted, each head's values repeated
    e = gpad3(q(kQX), 4, x, es, BL, 1, Dc, 0, 1, Dc, 0.0f, s);
    if (e == hipSuccess) e = repeat_f32(q(kQDelta), delta, es, BL * nheads, P, s);
    if (e == hipSuccess && z) e = gpad3(q(kQZ), 4, z, es, BL, 1, Dc, 0, 1, Dc, 0.0f, s);
    if (e == hipSuccess) e = gpad3(q(kQDy), 4, dy, es, BL, 1, Dc, 0, 1, Dc, 0.0f, s);
    if (e == hipSuccess) e = gpad3(q(kQB), 4, B, es, BL, 1, N, 0, 1, N, 0.0f, s);
    if (e == hipSuccess) e = gpad3(q(kQC), 4, C, es, BL, 1, N, 0, 1, N, 0.0f, s);
    if (e == hipSuccess) e = repeat_f32(q(kQA), A, 4, nheads, P * N, s);
    if (e == hipSuccess && Dskip) e = repeat_f32(q(kQD), Dskip, 4, nheads, P, s);
    if (e == hipSuccess && delta_bias) e = repeat_f32(q(kQBias), delta_bias, 4, nheads, P, s);
    if (e != hipSuccess) return hip_fail("ssd_bwd expansion launch", e);
    // the scan backward over the H * P channels (the Mamba discretisation: A_bar = exp(dt a_h),
    // B_bar = dt B), every input in fp32
    st = ssm_scan_bwd(batch, seqlen, Dc, N, SSM_DTYPE_F32, q(kQX), q(kQDelta), q(kQA), q(kQB), q(kQC),
                      Dskip ? q(kQD) : nullptr, z ? q(kQZ) : nullptr, h0, q(kQDy), dh_last, q(kQDx), q(kQDdelta),
                      q(kQDA), q(kQDB), q(kQDC), Dskip ? q(kQDD) : nullptr, z ? q(kQDz) : nullptr, dh0,
                      delta_softplus, SSM_DISC_MAMBA, delta_bias ? q(kQBias) : nullptr,
                      delta_bias ? q(kQDBias) : nullptr, nullptr, ws + off[kQInner], workspace_bytes - off[kQInner],
                      stream);
    if (st != SSM_OK) return st;
    // back to the layer's shapes: per-channel gradients converted, the tied ones summed over
    // each head's channels (in a fixed order)
    e = gunpad3(dx, es, q(kQDx), 4, BL, 1, Dc, 0, 1, Dc, s);
    if (e == hipSuccess && z) e = gunpad3(dz, es, q(kQDz), 4, BL, 1, Dc, 0, 1, Dc, s);
    if (e == hipSuccess) e = gunpad3(dB, es, q(kQDB), 4, BL, 1, N, 0, 1, N, s);
    if (e == hipSuccess) e = gunpad3(dC, es, q(kQDC), 4, BL, 1, N, 0, 1, N, s);
    if (e == hipSuccess) e = segsum(ddelta, es, q(kQDdelta), BL * nheads, P, s);
    if (e == hipSuccess) e = segsum(dA, 4, q(kQDA), nheads, P * N, s);
    if (e == hipSuccess && Dskip) e = segsum(dD, 4, q(kQDD), nheads, P, s);
    if (e == hipSuccess && delta_bias) e = segsum(ddelta_bias, 4, q(kQDBias), nheads, P, s);
    if (e != hipSuccess) return hip_fail("ssd_bwd reduction launch", e);
    return SSM_OK;
}
