// Host-side argument checks, launch planning and error text for libssm.
#include "ssm_host.h"

#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <initializer_list>

namespace ssm {

namespace {
thread_local char g_err[512] = {0};

constexpr int64_t kMaxElems = int64_t(1) << 50;  // keeps every byte offset far from int64 overflow

struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char *name, const void *p, int64_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool overlaps(const Range &a, const Range &b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int check_dims(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype) {
    if (dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16) {
        set_error("dtype %d is neither SSM_DTYPE_F32 (0) nor SSM_DTYPE_BF16 (1)", dtype);
        return SSM_EINVAL;
    }
    if (batch < 0 || seqlen < 0 || dim < 0) {
        set_error("negative size (batch=%lld seqlen=%lld dim=%lld)", (long long)batch,
                  (long long)seqlen, (long long)dim);
        return SSM_EINVAL;
    }
    if (dstate < 1) {
        set_error("dstate=%lld: need at least one state", (long long)dstate);
        return SSM_EINVAL;
    }
    if (dstate > SSM_MAX_DSTATE) {
        set_error("dstate=%lld exceeds the supported maximum %d", (long long)dstate, SSM_MAX_DSTATE);
        return SSM_EUNSUPPORTED;
    }
    // overflow-safe product checks
    if (batch > 0 && seqlen > 0 && dim > 0) {
        if (seqlen > kMaxElems / batch || dim > kMaxElems / (batch * seqlen) ||
            dstate > kMaxElems / (batch * seqlen)) {
            set_error("tensor of %lld x %lld x %lld elements is too large", (long long)batch,
                      (long long)seqlen, (long long)dim);
            return SSM_EINVAL;
        }
    }
    if (batch > 0 && dim > 0 && dim > kMaxElems / (batch * dstate)) {
        set_error("state of %lld x %lld x %lld elements is too large", (long long)batch,
                  (long long)dim, (long long)dstate);
        return SSM_EINVAL;
    }
    return SSM_OK;
}

int check_no_overlap(const Range *outs, int n_out, const Range *all, int n_all) {
    for (int i = 0; i < n_out; ++i)
        for (int j = 0; j < n_all; ++j) {
            if (outs[i].lo == all[j].lo && outs[i].hi == all[j].hi &&
                std::strcmp(outs[i].name, all[j].name) == 0)
                continue;  // itself
            if (overlaps(outs[i], all[j])) {
                set_error("output %s overlaps %s", outs[i].name, all[j].name);
                return SSM_EINVAL;
            }
        }
    return SSM_OK;
}

int check_aligned(const Range *all, int n) {
    for (int i = 0; i < n; ++i)
        if (all[i].lo && !aligned16(reinterpret_cast<const void *>(all[i].lo))) {
            set_error("pointer %s is not 16-byte aligned", all[i].name);
            return SSM_EINVAL;
        }
    return SSM_OK;
}
}  // namespace

bool env_flag(const char *name) {
    const char *v = std::getenv(name);
    return v && *v && std::strcmp(v, "0") != 0;
}

void log_call(const char *fmt, ...) {
    static const bool on = env_flag("SSM_LOG");
    if (!on) return;
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    std::fprintf(stderr, "[ssm] %s\n", buf);
}

void set_error(const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

void clear_error() { g_err[0] = 0; }

int plan_scan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
              const ssm_scan_opts *opts, ScanPlan *plan) {
    int st = check_dims(batch, seqlen, dim, dstate, dtype);
    if (st != SSM_OK) return st;
    ssm_scan_opts o{0, 0, 0, 0, 0};
    if (opts) o = *opts;
    if (o.one_block_per_cu < -1 || o.one_block_per_cu > 1) {
        set_error("opts.one_block_per_cu=%d must be -1, 0 or 1", o.one_block_per_cu);
        return SSM_EINVAL;
    }
    if (o.a_structure != 0 && o.a_structure != -1) {
        set_error("opts.a_structure=%d must be 0 or -1", o.a_structure);
        return SSM_EINVAL;
    }
    if (o.chunk_len < 0) {
        set_error("opts.chunk_len=%lld is negative", (long long)o.chunk_len);
        return SSM_EINVAL;
    }
    if (!(o.states_per_lane == 0 || o.states_per_lane == 1 || o.states_per_lane == 2 ||
          o.states_per_lane == 4 || o.states_per_lane == 8 || o.states_per_lane == 16)) {
        set_error("opts.states_per_lane=%d is not 0, 1, 2, 4, 8 or 16", o.states_per_lane);
        return SSM_EINVAL;
    }
    if (!(o.time_block == 0 || o.time_block == 8 || o.time_block == 16 || o.time_block == 32)) {
        set_error("opts.time_block=%d is not 0, 8, 16 or 32", o.time_block);
        return SSM_EINVAL;
    }
    ScanPlan p;
    // states per lane: default 4 (a quarter of the N=16 state in each of four waves); more
    // than 16 states take 16 per lane in up to 16 waves, with 8-step blocks
    int G = o.states_per_lane;
    if (dstate > 16) {
        if ((G != 0 && G != 16) || (o.time_block != 0 && o.time_block != 8)) {
            set_error("dstate=%lld > 16 runs 16 states per lane and 8-step blocks (opts asked %d, %d)",
                      (long long)dstate, G, o.time_block);
            return SSM_EINVAL;
        }
        G = 16;
    }
    if (G == 0) {
        G = 1;
        while (G < dstate && G < 4) G *= 2;
    }
    p.G = G;
    p.NW = static_cast<int>(ceil_div(dstate, G));
    // time block: each thread stages ceil(TB / NW) <= 8 rows, and the
    // workgroup's LDS (step sizes, B/C rows, per-wave y shares) stays <= 64 KiB
    auto rows_ok = [&](int tb) { return (tb + p.NW - 1) / p.NW <= 8; };
    auto lds_ok = [&](int tb) {
        const int64_t np = static_cast<int64_t>(p.NW) * p.G;
        return 4 * (tb * 64 * 2 + 2 * tb * np + static_cast<int64_t>(p.NW) * tb * 64) <= 65536;
    };
    if (o.time_block) {
        if (!rows_ok(o.time_block) || !lds_ok(o.time_block)) {
            set_error("opts.time_block=%d does not fit %d waves of %d states", o.time_block, p.NW, p.G);
            return SSM_EINVAL;
        }
        p.TB = o.time_block;
    } else {
        p.TB = 8;
        for (int tb : {32, 16}) {
            if (dstate <= 16 && rows_ok(tb) && lds_ok(tb)) {
                p.TB = tb;
                break;
            }
        }
    }
    const int64_t dblocks = ceil_div(dim, kChannelsPerBlock);
    const bool fast_ok = dstate == 16 && dim % 64 == 0 && dim < (int64_t(1) << 24) &&
                         (o.states_per_lane == 0 || o.states_per_lane == 2 || o.states_per_lane == 4) &&
                         (o.time_block == 0 || o.time_block == 16);
    // sequence chunks: split only when one pass leaves most SIMDs idle
    int64_t n_chunks = 1;
    if (seqlen > 0) {
        if (o.chunk_len > 0) {
            n_chunks = ceil_div(seqlen, o.chunk_len);
        } else if (fast_ok) {
            // specialised kernel: aim at one workgroup per CU (G = 2, two compute waves
            // per SIMD), the configuration with the highest update rate per CU
            const int64_t bd = batch * dblocks;
            const int64_t kMinChunk = 2048;   // keeps the carry pass's share small
            if (bd > 0 && bd < kCUs) {
                const int64_t want = ceil_div(kCUs, bd);
                const int64_t cap = ceil_div(seqlen, kMinChunk);
                n_chunks = want < cap ? want : cap;
                if (n_chunks < 1) n_chunks = 1;
            }
        } else if (dstate <= 16) {   // (more states: one pass; the chunked form needs opts)
            const int64_t waves = batch * dblocks * p.NW;
            const int64_t kSimds = 1024;      // 256 CUs x 4 SIMDs
            const int64_t kMinChunk = 2048;   // keeps the carry pass's share small
            if (waves > 0 && waves * 2 <= kSimds) {
                int64_t want = ceil_div(2 * kSimds, waves);
                int64_t cap = ceil_div(seqlen, kMinChunk);
                n_chunks = want < cap ? want : cap;
                if (n_chunks < 1) n_chunks = 1;
            }
        }
    }
    // a requested chunk length is kept as given (the last chunk takes the rest); the
    // planner's own count is balanced
    if (o.chunk_len > 0 && seqlen > 0) p.chunk_len = o.chunk_len < seqlen ? o.chunk_len : seqlen;
    else p.chunk_len = seqlen > 0 ? ceil_div(seqlen, n_chunks) : 0;
    p.n_chunks = seqlen > 0 ? ceil_div(seqlen, p.chunk_len > 0 ? p.chunk_len : 1) : 1;
    // grid: x = 64-channel blocks, y = batch rows, z = chunks (hardware limit 65535 on y and z)
    if (batch > 65535 || p.n_chunks > 65535 || dblocks > 0x7fffffff) {
        set_error("grid too large (batch=%lld, chunks=%lld): at most 65535 of each",
                  (long long)batch, (long long)p.n_chunks);
        return SSM_EUNSUPPORTED;
    }
    // specialised kernel: 16 / G compute waves (G = 2 or 4 states per lane) + 4 helper
    // waves, 16-step blocks, double-buffered LDS, B/C rows packed to fp32 by a pre-pass
    p.fast = fast_ok && (p.G == 2 || p.G == 4);
    if (p.fast) {
        // With G = 4 a grid of at most one compute wave per SIMD leaves each compute wave
        // alone on its SIMD, where it cannot hide the scalar-load latency of B/C; G = 2
        // puts two compute waves on every SIMD instead.
        const int64_t cw4 = batch * dblocks * p.n_chunks * 4;
        if (o.states_per_lane == 0) p.G = cw4 <= kCUs * 4 ? 2 : 4;
        p.TB = 16;
        p.NW = 16 / p.G + 4 + (p.G == 2 ? 1 : 0);   // compute, helper and prefetch waves
    }
    size_t ws = 0;
    if (p.n_chunks > 1) {
        const size_t carries = static_cast<size_t>(batch) * static_cast<size_t>(p.n_chunks - 1) *
                               static_cast<size_t>(dim);
        p.ws_P_off = 0;
        p.ws_H_off = align_up(carries * static_cast<size_t>(dstate) * sizeof(float), kWsAlign);
        ws = align_up(p.ws_H_off + carries * static_cast<size_t>(dstate) * sizeof(float), kWsAlign);
    }
    if (p.fast && p.n_chunks > 1 && p.chunk_len >= kLocalMinChunk) {
        // local-scan carries: every chunk's own end state, the partial sums of delta, flags
        p.local = true;
        const size_t bcdn = static_cast<size_t>(batch) * static_cast<size_t>(p.n_chunks) *
                            static_cast<size_t>(dim) * static_cast<size_t>(dstate);
        p.ws_Hl_off = ws;
        ws = align_up(ws + bcdn * sizeof(float), kWsAlign);
        p.ws_S_off = ws;
        ws = align_up(ws + 2 * static_cast<size_t>(batch) * static_cast<size_t>(p.n_chunks) * 8 *
                               static_cast<size_t>(dim) * sizeof(float), kWsAlign);
        p.ws_F_off = ws;
        ws = align_up(ws + static_cast<size_t>(batch) * static_cast<size_t>(p.n_chunks - 1) *
                               static_cast<size_t>(dim / 64) * sizeof(int), kWsAlign);
    }
    if (p.fast && seqlen > 0 && batch > 0 && dim > 0) {
        // [batch][chunks][bc_lpad/16][16/G][16/SUB][B, C][SUB][G] fp32 (SUB = 8/G), zero past
        // each chunk's end
        p.bc_lpad = ceil_div(p.chunk_len, 16) * 16;
        p.ws_BC_off = ws;
        ws = align_up(ws + static_cast<size_t>(batch) * static_cast<size_t>(p.n_chunks) *
                               static_cast<size_t>(p.bc_lpad) * 16 * 2 * sizeof(float),
                      kWsAlign);
    }
    p.structured = o.a_structure == 0;
    p.ws_bytes = ws;
    p.blocks = static_cast<uint64_t>(dblocks) * static_cast<uint64_t>(batch) *
               static_cast<uint64_t>(p.n_chunks);
    // With no more workgroups than CUs, the dispatcher may still stack two on one
    // CU and leave another idle; reserving over half of a CU's LDS prevents that.
    const bool one = o.one_block_per_cu == 1 ||
                     (o.one_block_per_cu == 0 && p.fast && p.blocks <= static_cast<uint64_t>(kCUs));
    if (one && p.fast) {
        // static LDS of the specialised kernel's y pass: double-buffered staging (TB/2 float4 per lane) and y shares (16/G waves)
        const size_t used = static_cast<size_t>(p.TB) * 1024 + static_cast<size_t>(16 / p.G) * p.TB * 512;
        if (used <= kLdsPerCU / 2) p.lds_reserve = kLdsPerCU / 2 + 1024 - used;
    }
    *plan = p;
    return SSM_OK;
}

namespace {
int check_variant(const ssm_variant *v) {
    if (!v) return SSM_OK;
    if (v->discretization < SSM_DISC_MAMBA || v->discretization > SSM_DISC_BILINEAR || v->reserved != 0) {
        set_error("variant.discretization=%d must be 0, 1 or 2 and variant.reserved 0", v->discretization);
        return SSM_EINVAL;
    }
    return SSM_OK;
}
}  // namespace

int check_scan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
               const void *x, const void *delta, const float *A, const void *B, const void *C,
               const float *Dskip, const void *z, const float *h0, const float *h_last,
               const void *y, int delta_softplus, const ssm_variant *variant,
               const ssm_scan_opts *opts, const void *workspace, size_t workspace_bytes,
               ScanPlan *plan) {
    int st = plan_scan(batch, seqlen, dim, dstate, dtype, opts, plan);
    if (st != SSM_OK) return st;
    if (delta_softplus != 0 && delta_softplus != 1) {
        set_error("delta_softplus=%d is neither 0 nor 1", delta_softplus);
        return SSM_EINVAL;
    }
    st = check_variant(variant);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;  // nothing to compute or store
    const int64_t es = static_cast<int64_t>(dtype_size(dtype));
    const int64_t tok = batch * seqlen * dim * es;
    const int64_t bc = batch * seqlen * dstate * es;
    const int64_t st_bytes = batch * dim * dstate * 4;
    if (seqlen > 0) {
        const char *missing = !x ? "x" : !delta ? "delta" : !A ? "A" : !B ? "B" : !C ? "C" : !y ? "y" : nullptr;
        if (missing) {
            set_error("required pointer %s is NULL", missing);
            return SSM_EINVAL;
        }
    }
    Range all[] = {
        range("x", x, tok),           range("delta", delta, tok),
        range("z", z, tok),           range("B", B, bc),
        range("C", C, bc),            range("A", A, dim * dstate * 4),
        range("Dskip", Dskip, dim * 4), range("h0", h0, st_bytes),
        range("h_last", h_last, st_bytes), range("y", y, seqlen > 0 ? tok : 0),
        range("workspace", workspace, static_cast<int64_t>(plan->ws_bytes)),
        range("delta_bias", variant_bias(variant), dim * 4),
    };
    const int n_all = static_cast<int>(sizeof(all) / sizeof(all[0]));
    st = check_aligned(all, n_all);
    if (st != SSM_OK) return st;
    Range outs[] = {all[9], all[8], all[10]};  // y, h_last, workspace
    st = check_no_overlap(outs, 3, all, n_all);
    if (st != SSM_OK) return st;
    if (plan->ws_bytes > 0) {
        if (!workspace || workspace_bytes < plan->ws_bytes) {
            set_error("workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0,
                      plan->ws_bytes);
            return SSM_EWORKSPACE;
        }
    }
    return SSM_OK;
}

int check_state_update(int64_t batch, int64_t dim, int64_t dstate, int dtype, const float *h,
                       const void *x, const void *delta, const float *A, const void *B,
                       const void *C, const float *Dskip, const void *z, const void *y,
                       int delta_softplus, const ssm_variant *variant) {
    int st = check_dims(batch, 1, dim, dstate, dtype);
    if (st != SSM_OK) return st;
    if (delta_softplus != 0 && delta_softplus != 1) {
        set_error("delta_softplus=%d is neither 0 nor 1", delta_softplus);
        return SSM_EINVAL;
    }
    st = check_variant(variant);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    if (batch * dim > (int64_t(1) << 34)) {   // 64 lanes per channel at most, 256-thread blocks
        set_error("batch*dim=%lld is too large for one launch", (long long)(batch * dim));
        return SSM_EUNSUPPORTED;
    }
    const char *missing = !h ? "h" : !x ? "x" : !delta ? "delta" : !A ? "A" : !B ? "B" : !C ? "C" : !y ? "y" : nullptr;
    if (missing) {
        set_error("required pointer %s is NULL", missing);
        return SSM_EINVAL;
    }
    const int64_t es = static_cast<int64_t>(dtype_size(dtype));
    Range all[] = {
        range("h", h, batch * dim * dstate * 4), range("x", x, batch * dim * es),
        range("delta", delta, batch * dim * es), range("z", z, batch * dim * es),
        range("B", B, batch * dstate * es),     range("C", C, batch * dstate * es),
        range("A", A, dim * dstate * 4),        range("Dskip", Dskip, dim * 4),
        range("y", y, batch * dim * es),        range("delta_bias", variant_bias(variant), dim * 4),
    };
    const int n_all = static_cast<int>(sizeof(all) / sizeof(all[0]));
    st = check_aligned(all, n_all);
    if (st != SSM_OK) return st;
    Range outs[] = {all[8], all[0]};  // y, h
    return check_no_overlap(outs, 2, all, n_all);
}

int plan_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                  BwdPlan *plan) {
    int st = check_dims(batch, seqlen, dim, dstate, dtype);
    if (st != SSM_OK) return st;
    if (dim >= (int64_t(1) << 24) - 64) {
        set_error("ssm_scan_bwd: dim=%lld is too large", (long long)dim);
        return SSM_EUNSUPPORTED;
    }
    if (dstate > 256) {
        set_error("ssm_scan_bwd supports dstate <= 256 (got %lld)", (long long)dstate);
        return SSM_EUNSUPPORTED;
    }
    if (dstate != 16 || dim % 64 != 0) {
        // run on copies padded to dim Dp and 16 states per group: the padding channels carry
        // x = 0, the padding states B = C = 0 (and A = -1), so neither adds to any gradient
        BwdPlan p;
        p.pad = true;
        p.Dp = ceil_div(dim, 64) * 64;
        p.K = ceil_div(dstate, 16);
        const int gdt = p.K > 1 ? SSM_DTYPE_F32 : dtype;   // the dtype the native kernels run in
        BwdPlan in;
        st = plan_scan_bwd(batch, seqlen, p.Dp, 16, gdt, &in);
        if (st != SSM_OK) return st;
        const size_t B = static_cast<size_t>(batch), L = static_cast<size_t>(seqlen);
        const size_t Dp = static_cast<size_t>(p.Dp), es = dtype_size(gdt);
        const size_t tok = B * L * Dp * es, bc = B * L * 16 * es, st16 = B * Dp * 16 * sizeof(float);
        // with several groups the token gradients go straight into the sums (no per-group copy);
        // fp32 tokens that need no padding are read in place and summed into the outputs
        p.direct = p.K > 1 && dtype == SSM_DTYPE_F32 && p.Dp == dim;
        const size_t tok_in = p.direct ? 0 : tok, tok_out = p.K > 1 ? 0 : tok;
        const size_t sum = (p.K > 1 && !p.direct) ? B * L * Dp * sizeof(float) : 0;
        const size_t bytes[kPadBufs] = {tok_in, tok_in, tok_in, tok_in, bc, bc, Dp * 16 * sizeof(float), Dp * sizeof(float),
                                        Dp * sizeof(float), st16, st16,
                                        tok_out, tok_out, tok_out, bc, bc, Dp * 16 * sizeof(float), Dp * sizeof(float),
                                        Dp * sizeof(float), st16,
                                        sum, sum, sum, p.K > 1 ? Dp * sizeof(float) : 0};
        size_t ws = 0;
        for (int i = 0; i < kPadBufs; ++i) {
            p.pad_off[i] = ws;
            ws = align_up(ws + bytes[i], kWsAlign);
        }
        p.inner_off = ws;
        p.nblk = in.nblk;
        p.n_chunks = in.n_chunks;
        p.chunk_len = in.chunk_len;
        p.ws_bytes = p.ws_bytes_saved = align_up(ws + in.ws_bytes, kWsAlign);
        p.ckpt_bytes = 0;
        if (batch == 0 || seqlen == 0 || dim == 0) p.ws_bytes = p.ws_bytes_saved = 0;
        *plan = p;
        return SSM_OK;
    }
    if (batch > 65535) {
        set_error("batch=%lld: at most 65535 rows", (long long)batch);
        return SSM_EUNSUPPORTED;
    }
    BwdPlan p;
    p.nblk = ceil_div(seqlen, 8);
    if (seqlen > 0) {
        // the forward planner's chunking (it splits the sequence when the channel blocks
        // alone leave most CUs idle), with the chunk length rounded up to a multiple of 16:
        // checkpoints sit every 8 steps from each chunk's start
        ScanPlan f0;
        st = plan_scan(batch, seqlen, dim, dstate, dtype, nullptr, &f0);
        if (st != SSM_OK) return st;
        const int64_t cl = f0.n_chunks > 1 ? ceil_div(ceil_div(seqlen, f0.n_chunks), 16) * 16 : seqlen;
        ssm_scan_opts o = {cl, 0, 0, 0, 0};
        st = plan_scan(batch, seqlen, dim, dstate, dtype, &o, &p.fwd);
        if (st != SSM_OK) return st;
        if (!p.fwd.fast || (p.fwd.n_chunks > 1 && p.fwd.chunk_len % 16 != 0)) {
            set_error("ssm_scan_bwd: no chunk plan for this shape");
            return SSM_EUNSUPPORTED;
        }
        p.n_chunks = p.fwd.n_chunks;
        p.chunk_len = p.fwd.chunk_len;
    }
    const size_t B = static_cast<size_t>(batch), L = static_cast<size_t>(seqlen), D = static_cast<size_t>(dim);
    const size_t NC = static_cast<size_t>(p.n_chunks);
    size_t ws = 0;
    p.partBC_off = ws;
    ws = align_up(ws + 2 * B * (D / 64) * L * 16 * sizeof(float), kWsAlign);
    p.partA_off = ws;
    ws = align_up(ws + NC * B * D * 16 * sizeof(float), kWsAlign);
    p.partD_off = ws;
    ws = align_up(ws + NC * B * 8 * D * sizeof(float), kWsAlign);
    p.partDB_off = ws;
    ws = align_up(ws + NC * B * 8 * D * sizeof(float), kWsAlign);
    if (p.n_chunks > 1) {
        const size_t carries = B * (NC - 1) * D * 16 * sizeof(float);
        p.lcP_off = ws;
        ws = align_up(ws + carries, kWsAlign);
        p.lcH_off = ws;
        ws = align_up(ws + carries, kWsAlign);
    }
    p.fwd_off = ws;
    p.ws_bytes_saved = ws;
    ws = align_up(ws + p.fwd.ws_bytes, kWsAlign);
    p.ckpt_off = ws;
    p.ckpt_bytes = B * static_cast<size_t>(p.nblk) * D * 16 * sizeof(float);
    ws = align_up(ws + p.ckpt_bytes, kWsAlign);
    p.ws_bytes = ws;
    if (batch == 0 || seqlen == 0 || dim == 0) p.ws_bytes = p.ws_bytes_saved = p.ckpt_bytes = 0;
    *plan = p;
    return SSM_OK;
}

int check_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                   const void *x, const void *delta, const float *A, const void *B, const void *C,
                   const float *Dskip, const void *z, const float *h0, const void *dy,
                   const float *dh_last, const void *dx, const void *ddelta, const float *dA,
                   const void *dB, const void *dC, const float *dD, const void *dz, const float *dh0,
                   int delta_softplus, int discretization, const float *delta_bias,
                   const float *ddelta_bias, const float *checkpoints,
                   const void *workspace, size_t workspace_bytes, BwdPlan *plan) {
    int st = plan_scan_bwd(batch, seqlen, dim, dstate, dtype, plan);
    if (st != SSM_OK) return st;
    if (plan->pad && checkpoints) {
        set_error("saved checkpoints need dstate == 16 and dim a multiple of 64 (got dstate=%lld, dim=%lld)",
                  (long long)dstate, (long long)dim);
        return SSM_EUNSUPPORTED;
    }
    if (delta_softplus != 0 && delta_softplus != 1) {
        set_error("delta_softplus=%d is neither 0 nor 1", delta_softplus);
        return SSM_EINVAL;
    }
    if (discretization < SSM_DISC_MAMBA || discretization > SSM_DISC_BILINEAR) {
        set_error("discretization=%d is not an ssm_discretization", discretization);
        return SSM_EINVAL;
    }
    // with batch == 0 the parameter gradients (dA, dD, ddelta_bias) are still written: zeros
    if (dim == 0) return SSM_OK;
    const char *missing = !A ? "A" : !dA ? "dA" : (z && !dz) ? "dz (z is given)" : (Dskip && !dD) ? "dD (Dskip is given)" :
                          (delta_bias && !ddelta_bias) ? "ddelta_bias (delta_bias is given)" : nullptr;
    if (!missing && seqlen > 0 && batch > 0)
        missing = !x ? "x" : !delta ? "delta" : !B ? "B" : !C ? "C" : !dy ? "dy" : !dx ? "dx" :
                  !ddelta ? "ddelta" : !dB ? "dB" : !dC ? "dC" : nullptr;
    if (missing) {
        set_error("required pointer %s is NULL", missing);
        return SSM_EINVAL;
    }
    const int64_t es = static_cast<int64_t>(dtype_size(dtype));
    const int64_t tok = batch * seqlen * dim * es;
    const int64_t bc = batch * seqlen * dstate * es;
    const int64_t stb = batch * dim * dstate * 4;
    Range all[] = {
        range("x", x, tok), range("delta", delta, tok), range("z", z, tok), range("B", B, bc),
        range("C", C, bc), range("A", A, dim * dstate * 4), range("Dskip", Dskip, dim * 4),
        range("h0", h0, stb), range("dy", dy, tok), range("dh_last", dh_last, stb),
        range("delta_bias", delta_bias, dim * 4),
        // outputs from here on
        range("dx", dx, tok), range("ddelta", ddelta, tok), range("dA", dA, dim * dstate * 4),
        range("dB", dB, bc), range("dC", dC, bc), range("dD", Dskip ? dD : nullptr, dim * 4),
        range("dz", z ? dz : nullptr, tok), range("dh0", dh0, stb),
        range("ddelta_bias", delta_bias ? ddelta_bias : nullptr, dim * 4),
        range("workspace", workspace, static_cast<int64_t>(checkpoints ? plan->ws_bytes_saved : plan->ws_bytes)),
        range("checkpoints", checkpoints, static_cast<int64_t>(plan->ckpt_bytes)),   // an input
    };
    const int n_all = static_cast<int>(sizeof(all) / sizeof(all[0]));
    st = check_aligned(all, n_all);
    if (st != SSM_OK) return st;
    st = check_no_overlap(all + 11, n_all - 12, all, n_all);
    if (st != SSM_OK) return st;
    const size_t need = checkpoints ? plan->ws_bytes_saved : plan->ws_bytes;
    if (seqlen > 0 && need > 0 && (!workspace || workspace_bytes < need)) {
        set_error("workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0, need);
        return SSM_EWORKSPACE;
    }
    return SSM_OK;
}

int check_scan_save(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                    const void *x, const void *delta, const float *A, const void *B, const void *C,
                    const float *Dskip, const void *z, const float *h0, const float *h_last,
                    const void *y, int delta_softplus, const ssm_variant *variant,
                    const float *checkpoints, const void *workspace, size_t workspace_bytes,
                    BwdPlan *plan) {
    int st = plan_scan_bwd(batch, seqlen, dim, dstate, dtype, plan);
    if (st != SSM_OK) return st;
    if (plan->pad) {
        set_error("ssm_scan_fwd_save supports dstate == 16 and dim a multiple of 64 (got dstate=%lld, dim=%lld)",
                  (long long)dstate, (long long)dim);
        return SSM_EUNSUPPORTED;
    }
    // the forward's own checks, on the backward's chunk plan (so that the checkpoints sit
    // every 8 steps from each chunk's start, as the reverse sweep reads them)
    ssm_scan_opts o = {plan->chunk_len, 0, 0, 0, 0};
    ScanPlan fp;
    st = check_scan(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, h_last, y,
                    delta_softplus, variant, seqlen > 0 ? &o : nullptr, workspace, workspace_bytes, &fp);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0 || seqlen == 0) return SSM_OK;
    if (fp.n_chunks != plan->fwd.n_chunks || fp.chunk_len != plan->fwd.chunk_len || !fp.fast) {
        set_error("ssm_scan_fwd_save: no chunk plan for this shape");
        return SSM_EUNSUPPORTED;
    }
    if (!checkpoints) {
        set_error("required pointer checkpoints is NULL");
        return SSM_EINVAL;
    }
    const int64_t es = static_cast<int64_t>(dtype_size(dtype));
    const int64_t tok = batch * seqlen * dim * es;
    const int64_t bc = batch * seqlen * dstate * es;
    const int64_t stb = batch * dim * dstate * 4;
    Range all[] = {
        range("checkpoints", checkpoints, static_cast<int64_t>(plan->ckpt_bytes)),
        range("x", x, tok), range("delta", delta, tok), range("z", z, tok), range("B", B, bc),
        range("C", C, bc), range("A", A, dim * dstate * 4), range("Dskip", Dskip, dim * 4),
        range("h0", h0, stb), range("h_last", h_last, stb), range("y", y, tok),
        range("workspace", workspace, static_cast<int64_t>(fp.ws_bytes)),
        range("delta_bias", variant_bias(variant), dim * 4),
    };
    const int n_all = static_cast<int>(sizeof(all) / sizeof(all[0]));
    st = check_aligned(all, 1);
    if (st != SSM_OK) return st;
    return check_no_overlap(all, 1, all, n_all);
}

namespace {
int check_conv_common(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int dtype, int silu) {
    if (dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16) {
        set_error("dtype=%d is neither SSM_DTYPE_F32 nor SSM_DTYPE_BF16", dtype);
        return SSM_EINVAL;
    }
    if (batch < 0 || seqlen < 0 || dim < 0) {
        set_error("negative size (batch=%lld, seqlen=%lld, dim=%lld)", (long long)batch, (long long)seqlen,
                  (long long)dim);
        return SSM_EINVAL;
    }
    if (width < 1) {
        set_error("width=%lld must be at least 1", (long long)width);
        return SSM_EINVAL;
    }
    if (width > 4) {
        set_error("width=%lld: at most 4 is supported", (long long)width);
        return SSM_EUNSUPPORTED;
    }
    if (silu != 0 && silu != 1) {
        set_error("silu=%d is neither 0 nor 1", silu);
        return SSM_EINVAL;
    }
    if (batch > 65535 || (seqlen + 31) / 32 > 65535 || (batch > 0 && dim > (int64_t(1) << 40) / (batch * (seqlen + 4)))) {
        set_error("shape too large for one launch (batch=%lld, seqlen=%lld, dim=%lld)", (long long)batch,
                  (long long)seqlen, (long long)dim);
        return SSM_EUNSUPPORTED;
    }
    return SSM_OK;
}
}  // namespace

int check_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int dtype,
                     const void *x, const float *w, const float *bias, const void *state_in,
                     const void *y, const void *state_out, int silu) {
    int st = check_conv_common(batch, seqlen, dim, width, dtype, silu);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    const char *missing = !w ? "w" : (seqlen > 0 && !x) ? "x" : (seqlen > 0 && !y) ? "y" : nullptr;
    if (missing) {
        set_error("required pointer %s is NULL", missing);
        return SSM_EINVAL;
    }
    const int64_t es = static_cast<int64_t>(dtype_size(dtype));
    const int64_t tok = batch * seqlen * dim * es;
    const int64_t stb = batch * dim * (width - 1) * es;
    Range all[] = {range("x", x, tok), range("w", w, dim * width * 4), range("bias", bias, dim * 4),
                   range("state_in", state_in, stb), range("y", y, tok), range("state_out", state_out, stb)};
    st = check_aligned(all, 6);
    if (st != SSM_OK) return st;
    return check_no_overlap(all + 4, 2, all, 6);
}

size_t conv1d_bwd_ws_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t width) {
    if (batch <= 0 || seqlen <= 0 || dim <= 0 || width < 1 || width > 4) return 0;
    const size_t tiles = static_cast<size_t>(ceil_div(seqlen, kConvBwdTile));
    return static_cast<size_t>(batch) * tiles * static_cast<size_t>(dim) * static_cast<size_t>(width + 1) *
           sizeof(float);
}

int check_conv1d_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int dtype,
                     const void *x, const float *w, const float *bias, const void *state_in,
                     const void *dy, const void *dx, const float *dw, const float *dbias,
                     const void *dstate, int silu, const void *workspace, size_t workspace_bytes) {
    int st = check_conv_common(batch, seqlen, dim, width, dtype, silu);
    if (st != SSM_OK) return st;
    if (ceil_div(seqlen, kConvBwdTile) > 65535 || batch > 65535) {
        set_error("grid too large (batch=%lld, seqlen=%lld): at most 65535 rows and 65535 x %d steps",
                  (long long)batch, (long long)seqlen, kConvBwdTile);
        return SSM_EUNSUPPORTED;
    }
    // with batch == 0 the filter gradients (dw, dbias) are still written: zeros
    if (dim == 0) return SSM_OK;
    const bool rows = seqlen > 0 && batch > 0;
    const char *missing = !w ? "w" : !dw ? "dw" : (rows && !x) ? "x" : (rows && !dy) ? "dy" : (rows && !dx) ? "dx" : nullptr;
    if (missing) {
        set_error("required pointer %s is NULL", missing);
        return SSM_EINVAL;
    }
    const int64_t es = static_cast<int64_t>(dtype_size(dtype));
    const int64_t tok = batch * seqlen * dim * es;
    const int64_t stb = batch * dim * (width - 1) * es;
    const size_t need = conv1d_bwd_ws_bytes(batch, seqlen, dim, width);
    Range all[] = {range("x", x, tok), range("w", w, dim * width * 4), range("bias", bias, dim * 4),
                   range("state_in", state_in, stb), range("dy", dy, tok),
                   // outputs from here on
                   range("dx", dx, tok), range("dw", dw, dim * width * 4), range("dbias", dbias, dim * 4),
                   range("dstate", width > 1 ? dstate : nullptr, stb),
                   range("workspace", workspace, static_cast<int64_t>(need))};
    st = check_aligned(all, 10);
    if (st != SSM_OK) return st;
    st = check_no_overlap(all + 5, 5, all, 10);
    if (st != SSM_OK) return st;
    if (need > 0 && (!workspace || workspace_bytes < need)) {
        set_error("workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0, need);
        return SSM_EWORKSPACE;
    }
    return SSM_OK;
}

int check_conv1d_update(int64_t batch, int64_t dim, int64_t width, int dtype, const void *state,
                        const void *x, const float *w, const float *bias, const void *y, int silu) {
    int st = check_conv_common(batch, 1, dim, width, dtype, silu);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    const char *missing = !w ? "w" : !x ? "x" : !y ? "y" : (width > 1 && !state) ? "state" : nullptr;
    if (missing) {
        set_error("required pointer %s is NULL", missing);
        return SSM_EINVAL;
    }
    const int64_t es = static_cast<int64_t>(dtype_size(dtype));
    Range all[] = {range("x", x, batch * dim * es), range("w", w, dim * width * 4), range("bias", bias, dim * 4),
                   range("state", state, batch * dim * (width - 1) * es), range("y", y, batch * dim * es)};
    st = check_aligned(all, 5);
    if (st != SSM_OK) return st;
    return check_no_overlap(all + 3, 2, all, 5);
}

int check_ssd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups, int dtype,
              const void *x, const void *delta, const float *A, const void *B, const void *C,
              const float *Dskip, const void *z, const float *delta_bias, const float *h0,
              const float *h_last, const void *y, int delta_softplus) {
    if (dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16) {
        set_error("dtype %d is neither SSM_DTYPE_F32 (0) nor SSM_DTYPE_BF16 (1)", dtype);
        return SSM_EINVAL;
    }
    if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 1 || dstate < 1) {
        set_error("bad size (batch=%lld seqlen=%lld nheads=%lld headdim=%lld dstate=%lld)", (long long)batch,
                  (long long)seqlen, (long long)nheads, (long long)headdim, (long long)dstate);
        return SSM_EINVAL;
    }
    if (delta_softplus != 0 && delta_softplus != 1) {
        set_error("delta_softplus=%d is neither 0 nor 1", delta_softplus);
        return SSM_EINVAL;
    }
    if (ngroups < 1 || (nheads > 0 && nheads % ngroups != 0)) {
        set_error("ngroups=%lld must be >= 1 and divide nheads=%lld", (long long)ngroups, (long long)nheads);
        return SSM_EINVAL;
    }
    if (dstate > SSM_MAX_DSTATE) {
        set_error("the SSD scan supports dstate <= %d (got %lld)", SSM_MAX_DSTATE, (long long)dstate);
        return SSM_EUNSUPPORTED;
    }
    const bool mfma = headdim == 64 && dstate == 128 && dtype == SSM_DTYPE_BF16;
    if (!mfma && ngroups > 1 && ((nheads / ngroups) * headdim) % 64 != 0) {
        // the generic kernel stages one B/C row per 64-channel workgroup
        set_error("with ngroups=%lld each group's %lld channels must be a multiple of 64 (head dim %lld, "
                  "dstate %lld, dtype %d)", (long long)ngroups, (long long)((nheads / ngroups) * headdim),
                  (long long)headdim, (long long)dstate, dtype);
        return SSM_EUNSUPPORTED;
    }
    if (nheads > 0 && headdim > (int64_t(1) << 24) / nheads) {
        set_error("nheads * headdim = %lld * %lld is too large", (long long)nheads, (long long)headdim);
        return SSM_EUNSUPPORTED;
    }
    if (batch > 0 && seqlen > 0 && nheads > 0 &&
        (seqlen > kMaxElems / batch || nheads * headdim > kMaxElems / (batch * seqlen))) {
        set_error("tensor of %lld x %lld x %lld x %lld elements is too large", (long long)batch,
                  (long long)seqlen, (long long)nheads, (long long)headdim);
        return SSM_EINVAL;
    }
    if (batch * nheads > (int64_t(1) << 31)) {
        set_error("batch*nheads=%lld exceeds one launch", (long long)(batch * nheads));
        return SSM_EUNSUPPORTED;
    }
    if (batch == 0 || nheads == 0) return SSM_OK;
    const char *missing = !A ? "A" : (seqlen > 0 && !x) ? "x" : (seqlen > 0 && !delta) ? "delta"
                        : (seqlen > 0 && !B) ? "B" : (seqlen > 0 && !C) ? "C" : (seqlen > 0 && !y) ? "y" : nullptr;
    if (missing) {
        set_error("required pointer %s is NULL", missing);
        return SSM_EINVAL;
    }
    const int64_t es = static_cast<int64_t>(dtype_size(dtype));
    const int64_t tok = batch * seqlen * nheads * headdim * es;
    const int64_t st_bytes = batch * nheads * headdim * dstate * 4;
    Range all[] = {
        range("x", x, tok), range("delta", delta, batch * seqlen * nheads * es), range("A", A, nheads * 4),
        range("B", B, batch * seqlen * ngroups * dstate * es), range("C", C, batch * seqlen * ngroups * dstate * es),
        range("Dskip", Dskip, nheads * 4), range("z", z, tok), range("delta_bias", delta_bias, nheads * 4),
        range("h0", h0, st_bytes), range("h_last", h_last, st_bytes), range("y", y, seqlen > 0 ? tok : 0),
    };
    const int n_all = static_cast<int>(sizeof(all) / sizeof(all[0]));
    int st = check_aligned(all, n_all);
    if (st != SSM_OK) return st;
    return check_no_overlap(all + 9, 2, all, n_all);   // h_last, y
}

}  // namespace ssm

extern "C" {

size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                                    int saved_checkpoints) {
    ssm::clear_error();
    ssm::BwdPlan p;
    if (ssm::plan_scan_bwd(batch, seqlen, dim, dstate, dtype, &p) != SSM_OK) return 0;
    return saved_checkpoints ? p.ws_bytes_saved : p.ws_bytes;
}

int ssm_scan_save_sizes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                        size_t *workspace_bytes, size_t *checkpoint_bytes) {
    ssm::clear_error();
    if (!workspace_bytes || !checkpoint_bytes) {
        ssm::set_error("required pointer %s is NULL", !workspace_bytes ? "workspace_bytes" : "checkpoint_bytes");
        return SSM_EINVAL;
    }
    *workspace_bytes = 0;
    *checkpoint_bytes = 0;
    ssm::BwdPlan p;
    const int st = ssm::plan_scan_bwd(batch, seqlen, dim, dstate, dtype, &p);
    if (st != SSM_OK) return st;
    if (p.pad) {
        ssm::set_error("ssm_scan_fwd_save supports dstate == 16 and dim a multiple of 64 (got dstate=%lld, dim=%lld)",
                       (long long)dstate, (long long)dim);
        return SSM_EUNSUPPORTED;
    }
    if (batch > 0 && seqlen > 0 && dim > 0) *workspace_bytes = p.fwd.ws_bytes;
    *checkpoint_bytes = p.ckpt_bytes;
    return SSM_OK;
}

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char *ssm_status_str(int status) {
    switch (status) {
        case SSM_OK: return "ok";
        case SSM_EINVAL: return "invalid argument";
        case SSM_EUNSUPPORTED: return "unsupported";
        case SSM_EWORKSPACE: return "workspace too small";
        case SSM_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *ssm_last_error(void) { return ssm::g_err; }

int ssm_scan_plan_get(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                      const ssm_scan_opts *opts, ssm_scan_plan *out) {
    ssm::clear_error();
    if (!out) {
        ssm::set_error("plan pointer is NULL");
        return SSM_EINVAL;
    }
    ssm::ScanPlan p;
    int st = ssm::plan_scan(batch, seqlen, dim, dstate, dtype, opts, &p);
    if (st != SSM_OK) return st;
    std::memset(out, 0, sizeof(*out));
    out->chunk_len = p.chunk_len;
    out->n_chunks = p.n_chunks;
    out->states_per_lane = p.G;
    out->waves_per_block = p.NW;
    out->time_block = p.TB;
    out->specialised = p.fast ? 1 : 0;
    out->workspace_bytes = p.ws_bytes;
    out->lds_reserve = p.lds_reserve;
    out->blocks = p.blocks;
    return SSM_OK;
}

size_t ssm_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                int dtype, const ssm_scan_opts *opts) {
    ssm::ScanPlan p;
    if (ssm::plan_scan(batch, seqlen, dim, dstate, dtype, opts, &p) != SSM_OK) return 0;
    return p.ws_bytes;
}

}  // extern "C"
