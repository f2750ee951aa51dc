// Drives every argument-check path of libssm's host layer (built with g++
// under AddressSanitizer + UndefinedBehaviorSanitizer; no GPU, no HIP).
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <initializer_list>

#include "ssm.h"
#include "ssm_host.h"

static int fails = 0;
#define EXPECT(cond)                                                      \
    do {                                                                  \
        if (!(cond)) {                                                    \
            std::printf("FAIL line %d: %s (%s)\n", __LINE__, #cond, ssm_last_error()); \
            ++fails;                                                      \
        }                                                                 \
    } while (0)

static void *P(uintptr_t a) { return reinterpret_cast<void *>(a); }

int main() {
    using namespace ssm;
    ScanPlan p;
    // fake, well-separated, 16-byte aligned device addresses (never dereferenced)
    const uintptr_t base = uintptr_t(1) << 40, gap = uintptr_t(1) << 32;
    void *x = P(base), *dl = P(base + gap), *z = P(base + 2 * gap), *B = P(base + 3 * gap),
         *C = P(base + 4 * gap), *y = P(base + 5 * gap), *ws = P(base + 9 * gap);
    float *A = static_cast<float *>(P(base + 6 * gap)), *Dk = static_cast<float *>(P(base + 7 * gap));
    float *h0 = static_cast<float *>(P(base + 8 * gap)), *hl = static_cast<float *>(P(base + 10 * gap));
    auto scan = [&](int64_t b, int64_t l, int64_t d, int64_t n, int dt, const void *x_, const void *y_,
                    const ssm_scan_opts *o, const void *w, size_t wb, const float *h0_, const float *hl_) {
        return check_scan(b, l, d, n, dt, x_, dl, A, B, C, Dk, z, h0_, hl_, y_, 0, nullptr, o, w, wb, &p);
    };
    // discretisation variants and the delta bias
    {
        float *bias = static_cast<float *>(P(base + 11 * gap));
        const ssm_variant ok1{SSM_DISC_ZOH, 0, bias}, ok2{SSM_DISC_BILINEAR, 0, nullptr};
        const ssm_variant bad1{3, 0, nullptr}, bad2{-1, 0, nullptr}, bad3{SSM_DISC_ZOH, 1, nullptr};
        const ssm_variant mis{SSM_DISC_MAMBA, 0, static_cast<float *>(P(base + 11 * gap + 4))};
        const ssm_variant ovl{SSM_DISC_MAMBA, 0, static_cast<float *>(y)};
        auto sv = [&](const ssm_variant *v) {
            return check_scan(4, 256, 4096, 16, 1, x, dl, A, B, C, Dk, z, h0, hl, y, 1, v, nullptr, ws,
                              size_t(1) << 30, &p);
        };
        EXPECT(sv(&ok1) == SSM_OK);
        EXPECT(sv(&ok2) == SSM_OK);
        EXPECT(sv(&bad1) == SSM_EINVAL);
        EXPECT(sv(&bad2) == SSM_EINVAL);
        EXPECT(sv(&bad3) == SSM_EINVAL);
        EXPECT(sv(&mis) == SSM_EINVAL);
        EXPECT(std::strstr(ssm_last_error(), "delta_bias") != nullptr);
        EXPECT(sv(&ovl) == SSM_EINVAL);
        EXPECT(check_state_update(256, 4096, 16, 1, h0, x, dl, A, B, C, Dk, z, y, 0, &ok1) == SSM_OK);
        EXPECT(check_state_update(256, 4096, 16, 1, h0, x, dl, A, B, C, Dk, z, y, 0, &bad1) == SSM_EINVAL);
        EXPECT(check_state_update(256, 4096, 16, 1, h0, x, dl, A, B, C, Dk, z, y, 0, &mis) == SSM_EINVAL);
    }
    // backward: the delta bias needs its gradient output, aligned and apart from the others
    {
        BwdPlan bp;
        void *dx = P(base + 12 * gap), *ddl = P(base + 13 * gap), *dB = P(base + 14 * gap), *dC = P(base + 15 * gap);
        float *dA = static_cast<float *>(P(base + 16 * gap)), *dD = static_cast<float *>(P(base + 17 * gap));
        void *dz = P(base + 18 * gap), *dy = P(base + 19 * gap), *bws = P(base + 20 * gap);
        float *bias = static_cast<float *>(P(base + 21 * gap)), *dbias = static_cast<float *>(P(base + 22 * gap));
        auto bw = [&](const float *bi, const float *dbi, int disc = SSM_DISC_MAMBA, const float *ck = nullptr,
                      size_t wsb = size_t(1) << 30) {
            return check_scan_bwd(2, 1000, 256, 16, SSM_DTYPE_BF16, x, dl, A, B, C, Dk, z, nullptr, dy, nullptr,
                                  dx, ddl, dA, dB, dC, dD, dz, nullptr, 1, disc, bi, dbi, ck, bws, wsb, &bp);
        };
        EXPECT(bw(nullptr, nullptr) == SSM_OK);
        EXPECT(bw(nullptr, nullptr, SSM_DISC_ZOH) == SSM_OK);
        EXPECT(bw(bias, dbias, SSM_DISC_BILINEAR) == SSM_OK);
        EXPECT(bw(nullptr, nullptr, 3) == SSM_EINVAL);
        EXPECT(std::strstr(ssm_last_error(), "discretization") != nullptr);
        EXPECT(bw(nullptr, nullptr, -1) == SSM_EINVAL);
        EXPECT(bw(bias, dbias) == SSM_OK);
        EXPECT(bp.partDB_off > bp.partD_off && bp.ws_bytes >= bp.partDB_off + size_t(2) * 8 * 256 * 4);
        EXPECT(bw(nullptr, dbias) == SSM_OK);    // ignored without a bias
        EXPECT(bw(bias, nullptr) == SSM_EINVAL);
        EXPECT(std::strstr(ssm_last_error(), "ddelta_bias") != nullptr);
        EXPECT(bw(static_cast<float *>(P(base + 21 * gap + 4)), dbias) == SSM_EINVAL);
        EXPECT(bw(bias, static_cast<float *>(dx)) == SSM_EINVAL);    // overlaps dx
        EXPECT(std::strstr(ssm_last_error(), "overlaps") != nullptr);
        EXPECT(bw(bias, bias) == SSM_EINVAL);                        // output on an input
        // chunking: one chunk when the channel blocks fill the GPU; otherwise the forward
        // planner's count, chunks a multiple of 16 steps, and the adjoint carries
        EXPECT(plan_scan_bwd(4, 4096, 4096, 16, SSM_DTYPE_BF16, &bp) == SSM_OK);
        EXPECT(bp.n_chunks == 1 && bp.chunk_len == 4096 && bp.lcP_off == 0 && bp.fwd.n_chunks == 1);
        EXPECT(plan_scan_bwd(2, 1001, 256, 16, SSM_DTYPE_F32, &bp) == SSM_OK);
        EXPECT(bp.n_chunks == 1 && bp.chunk_len == 1001 && bp.nblk == 126);
        EXPECT(plan_scan_bwd(1, 5000, 128, 16, SSM_DTYPE_BF16, &bp) == SSM_OK);
        EXPECT(bp.n_chunks == 3 && bp.chunk_len == 1680 && bp.fwd.chunk_len == 1680 && bp.fwd.n_chunks == 3);
        EXPECT(bp.lcH_off > bp.lcP_off && bp.lcP_off > bp.partDB_off && bp.ws_bytes >= bp.lcH_off + size_t(2) * 128 * 16 * 4);
        EXPECT(plan_scan_bwd(1, 1048576, 1024, 16, SSM_DTYPE_BF16, &bp) == SSM_OK);
        EXPECT(bp.n_chunks == 16 && bp.chunk_len == 65536 && bp.nblk == 131072);
        EXPECT(bp.fwd.ws_bytes > 0 && bp.ckpt_off >= bp.fwd.ws_bytes);
        // saved checkpoints: the checkpoint pass's regions sit last, so the call given them
        // needs only the part before them
        EXPECT(bp.ws_bytes_saved == bp.fwd_off && bp.ckpt_off >= bp.fwd_off + bp.fwd.ws_bytes);
        EXPECT(bp.ckpt_bytes == size_t(1) * 131072 * 16 * 1024 * 4 && bp.ws_bytes >= bp.ckpt_off + bp.ckpt_bytes);
        float *ck = static_cast<float *>(P(base + 23 * gap));
        EXPECT(plan_scan_bwd(2, 1000, 256, 16, SSM_DTYPE_BF16, &bp) == SSM_OK);
        const size_t saved = bp.ws_bytes_saved, full = bp.ws_bytes;
        EXPECT(saved < full && bp.ckpt_bytes == size_t(2) * 125 * 16 * 256 * 4);
        EXPECT(bw(nullptr, nullptr, SSM_DISC_MAMBA, ck, saved) == SSM_OK);
        EXPECT(bw(nullptr, nullptr, SSM_DISC_MAMBA, nullptr, saved) == SSM_EWORKSPACE);
        EXPECT(bw(nullptr, nullptr, SSM_DISC_MAMBA, ck, saved - 1) == SSM_EWORKSPACE);
        EXPECT(bw(nullptr, nullptr, SSM_DISC_MAMBA, static_cast<float *>(dx), full) == SSM_EINVAL);   // dx on it
        EXPECT(std::strstr(ssm_last_error(), "overlaps") != nullptr);
        EXPECT(bw(nullptr, nullptr, SSM_DISC_MAMBA, static_cast<float *>(P(base + 23 * gap + 8)), full) == SSM_EINVAL);
        // the forward that stores them: the forward's checks on the backward's chunks
        void *sy = P(base + 24 * gap);
        auto sv = [&](int64_t Bn, int64_t Ln, int64_t Dn, int64_t Nn, float *c, void *yy, size_t wsb) {
            return check_scan_save(Bn, Ln, Dn, Nn, SSM_DTYPE_BF16, x, dl, A, B, C, Dk, z, nullptr, nullptr, yy, 0,
                                   nullptr, c, bws, wsb, &bp);
        };
        EXPECT(sv(2, 1000, 256, 16, ck, sy, size_t(1) << 30) == SSM_OK);
        EXPECT(bp.n_chunks == 1 && bp.fwd.fast);
        EXPECT(sv(2, 1000, 256, 16, nullptr, sy, size_t(1) << 30) == SSM_EINVAL);
        EXPECT(sv(2, 1000, 256, 16, ck, sy, 0) == SSM_EWORKSPACE);            // packed B/C rows
        EXPECT(sv(2, 1000, 256, 16, static_cast<float *>(sy), sy, size_t(1) << 30) == SSM_EINVAL);
        EXPECT(sv(2, 1000, 256, 12, ck, sy, size_t(1) << 30) == SSM_EUNSUPPORTED);
        EXPECT(sv(2, 1000, 96, 16, ck, sy, size_t(1) << 30) == SSM_EUNSUPPORTED);
        EXPECT(sv(1, 5000, 128, 16, ck, sy, size_t(1) << 30) == SSM_OK);
        EXPECT(bp.n_chunks == 3 && bp.fwd.chunk_len == 1680);
        size_t wsz = 1, ckz = 1;
        EXPECT(ssm_scan_save_sizes(1, 5000, 128, 16, SSM_DTYPE_BF16, &wsz, &ckz) == SSM_OK);
        EXPECT(wsz == bp.fwd.ws_bytes && ckz == size_t(625) * 16 * 128 * 4);
        EXPECT(ssm_scan_save_sizes(1, 5000, 96, 16, SSM_DTYPE_BF16, &wsz, &ckz) == SSM_EUNSUPPORTED && wsz == 0);
        EXPECT(ssm_scan_save_sizes(1, 5000, 128, 16, SSM_DTYPE_BF16, nullptr, &ckz) == SSM_EINVAL);
        EXPECT(ssm_scan_bwd_workspace_bytes(2, 1000, 256, 16, SSM_DTYPE_BF16, 1) == saved);
        EXPECT(ssm_scan_bwd_workspace_bytes(2, 1000, 256, 16, SSM_DTYPE_BF16, 0) == full);
        // other shapes: the native plan of the copies padded to 64 channels and 16 states,
        // after the padded buffers; no saved checkpoints
        BwdPlan in;
        EXPECT(plan_scan_bwd(2, 100, 40, 8, SSM_DTYPE_BF16, &bp) == SSM_OK);
        EXPECT(plan_scan_bwd(2, 100, 64, 16, SSM_DTYPE_BF16, &in) == SSM_OK);
        EXPECT(bp.pad && bp.Dp == 64 && !in.pad && bp.nblk == in.nblk);
        EXPECT(bp.pad_off[kPDx] >= size_t(4) * 2 * 100 * 64 * 2 && bp.inner_off > bp.pad_off[kPDh0]);
        EXPECT(bp.ws_bytes >= bp.inner_off + in.ws_bytes && bp.ws_bytes_saved == bp.ws_bytes);
        EXPECT(ssm_scan_bwd_workspace_bytes(2, 100, 40, 8, SSM_DTYPE_BF16, 0) == bp.ws_bytes);
        EXPECT(plan_scan_bwd(1, 10, 128, 3, SSM_DTYPE_F32, &bp) == SSM_OK && bp.pad && bp.Dp == 128);
        EXPECT(plan_scan_bwd(1, 10, 128, 257, SSM_DTYPE_F32, &bp) == SSM_EUNSUPPORTED);
        // more than 16 states: groups of 16 on fp32 copies, with fp32 sums of the per-channel
        // gradients after the outputs
        EXPECT(plan_scan_bwd(2, 100, 40, 40, SSM_DTYPE_BF16, &bp) == SSM_OK && bp.pad && bp.K == 3 && bp.Dp == 64);
        EXPECT(bp.pad_off[kPDx] >= size_t(4) * 2 * 100 * 64 * 4 && bp.pad_off[kSDx] > bp.pad_off[kPDh0]);
        EXPECT(bp.pad_off[kSDBias] >= bp.pad_off[kSDz] + size_t(2) * 100 * 64 * 4 && bp.inner_off > bp.pad_off[kSDBias]);
        EXPECT(plan_scan_bwd(2, 100, 40, 8, SSM_DTYPE_BF16, &bp) == SSM_OK && bp.K == 1);
        EXPECT(check_scan_bwd(2, 100, 40, 8, SSM_DTYPE_BF16, x, dl, A, B, C, nullptr, nullptr, nullptr, dl, nullptr,
                              dx, ddl, dA, dB, dC, nullptr, nullptr, nullptr, 0, SSM_DISC_MAMBA, nullptr,
                              nullptr, ck, bws, size_t(1) << 30, &bp) == SSM_EUNSUPPORTED);
        EXPECT(std::strstr(ssm_last_error(), "checkpoints") != nullptr);
    }
    // the specialised path packs B/C rows into the workspace: 4 x 4096 x 16 x (B, C) fp32
    EXPECT(scan(4, 4096, 4096, 16, SSM_DTYPE_BF16, x, y, nullptr, nullptr, 0, h0, hl) == SSM_EWORKSPACE);
    EXPECT(scan(4, 4096, 4096, 16, SSM_DTYPE_BF16, x, y, nullptr, ws, size_t(1) << 30, h0, hl) == SSM_OK);
    EXPECT(p.n_chunks == 1 && p.G == 2 && p.NW == 13 && p.TB == 16 && p.fast);
    EXPECT(p.ws_bytes == size_t(4) * 4096 * 16 * 2 * 4 && p.bc_lpad == 4096);
    EXPECT(p.lds_reserve + 16384 + 2 * (16 / p.G) * 4096 > 80 * 1024 && p.lds_reserve + 16384 + 2 * (16 / p.G) * 4096 <= 160 * 1024);
    EXPECT(scan(4, 4096, 4096, 16, 2, x, y, nullptr, ws, size_t(1) << 30, h0, hl) == SSM_EINVAL);
    EXPECT(scan(4, 4096, 4096, 257, 1, x, y, nullptr, ws, size_t(1) << 30, h0, hl) == SSM_EUNSUPPORTED);
    // more than 16 states: the generic kernel, 16 states per lane, 8-step blocks, one pass
    EXPECT(scan(4, 4096, 64, 17, 1, x, y, nullptr, ws, size_t(1) << 30, h0, hl) == SSM_OK);
    EXPECT(!p.fast && p.G == 16 && p.NW == 2 && p.TB == 8 && p.n_chunks == 1);
    EXPECT(scan(1, 4096, 64, 256, 1, x, y, nullptr, ws, size_t(1) << 30, h0, hl) == SSM_OK);
    EXPECT(!p.fast && p.G == 16 && p.NW == 16 && p.TB == 8 && p.n_chunks == 1);
    EXPECT(scan(4, 4096, 4096, 0, 1, x, y, nullptr, ws, size_t(1) << 30, h0, hl) == SSM_EINVAL);
    EXPECT(scan(-1, 4096, 4096, 16, 1, x, y, nullptr, ws, size_t(1) << 30, h0, hl) == SSM_EINVAL);
    EXPECT(scan(4, 4096, 4096, 16, 1, nullptr, y, nullptr, ws, size_t(1) << 30, h0, hl) == SSM_EINVAL);
    EXPECT(scan(4, 4096, 4096, 16, 1, P(base + 2), y, nullptr, ws, size_t(1) << 30, h0, hl) == SSM_EINVAL);
    EXPECT(scan(4, 4096, 4096, 16, 1, x, P(base + 64), nullptr, ws, size_t(1) << 30, h0, hl) == SSM_EINVAL);
    EXPECT(std::strstr(ssm_last_error(), "overlaps") != nullptr);
    EXPECT(scan(4, 4096, 4096, 16, 1, x, y, nullptr, ws, size_t(1) << 30, h0, h0) == SSM_EINVAL);
    EXPECT(scan(int64_t(1) << 30, int64_t(1) << 30, 4096, 16, 1, x, y, nullptr, nullptr, 0, h0, hl) == SSM_EINVAL);
    // empty problems are valid no-ops, even with null data pointers
    EXPECT(scan(0, 4096, 4096, 16, 1, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr) == SSM_OK);
    EXPECT(scan(4, 0, 4096, 16, 1, nullptr, nullptr, nullptr, nullptr, 0, h0, hl) == SSM_OK);
    // chunked plan needs a workspace
    ssm_scan_opts o{1024, 0, 0, 0, 0};
    EXPECT(scan(1, 8192, 1024, 16, 1, x, y, &o, nullptr, 0, h0, hl) == SSM_EWORKSPACE);
    EXPECT(p.n_chunks == 8 && p.ws_bytes > 0 && p.ws_BC_off > p.ws_H_off && p.bc_lpad == 1024);
    EXPECT(p.ws_P_off == 0 && p.ws_H_off == size_t(7) * 1024 * 16 * 4);   // per-state chunk decays, then end states
    const size_t need = p.ws_bytes;
    EXPECT(scan(1, 8192, 1024, 16, 1, x, y, &o, ws, need - 1, h0, hl) == SSM_EWORKSPACE);
    EXPECT(scan(1, 8192, 1024, 16, 1, x, y, &o, ws, need, h0, hl) == SSM_OK);
    EXPECT(ssm_scan_workspace_bytes(1, 8192, 1024, 16, 1, &o) == need);
    ssm_scan_opts bad1{-5, 0, 0, 0, 0}, bad2{0, 3, 0, 0, 0}, bad3{0, 0, 24, 0, 0}, bad4{0, 1, 32, 0, 0}, bad5{0, 0, 0, 2, 0};
    EXPECT(scan(1, 100, 64, 16, 1, x, y, &bad1, nullptr, 0, h0, hl) == SSM_EINVAL);
    EXPECT(scan(1, 100, 64, 16, 1, x, y, &bad2, nullptr, 0, h0, hl) == SSM_EINVAL);
    EXPECT(scan(1, 100, 64, 16, 1, x, y, &bad3, nullptr, 0, h0, hl) == SSM_EINVAL);
    EXPECT(scan(1, 100, 64, 16, 1, x, y, &bad4, nullptr, 0, h0, hl) == SSM_EINVAL);
    EXPECT(scan(1, 100, 64, 16, 1, x, y, &bad5, nullptr, 0, h0, hl) == SSM_EINVAL);
    // automatic chunking for a long, narrow sequence
    EXPECT(scan(1, int64_t(1) << 20, 1024, 16, 1, x, y, nullptr, ws, size_t(1) << 30, h0, hl) == SSM_OK);
    EXPECT(p.n_chunks > 1);
    // every plan keeps the staging and LDS limits the kernel relies on
    for (int n = 1; n <= 16; ++n)
        for (int g : {0, 1, 2, 4, 8, 16}) {
            ssm_scan_opts og{0, g, 0, 0, 0};
            if (plan_scan(3, 1000, n == 16 ? 128 : 100, n, 1, &og, &p) != SSM_OK) { EXPECT(false); continue; }
            if (p.fast) {   // 16/G compute waves + 4 helpers, double-buffered staging and y shares
                EXPECT(n == 16 && p.NW == 16 / p.G + 4 + (p.G == 2) && (p.G == 2 || p.G == 4) && p.TB == 16);
                continue;
            }
            const int rows = (p.TB + p.NW - 1) / p.NW;
            EXPECT(rows <= 8);
            EXPECT(p.NW * p.G >= n && p.NW * p.G <= 16 && p.NW * 64 <= 1024);
            EXPECT(4 * (p.TB * 128 + 2 * p.TB * p.NW * p.G + p.NW * p.TB * 64) <= 65536);
        }
    // state update
    float *h = h0;
    EXPECT(check_state_update(256, 4096, 16, 1, h, x, dl, A, B, C, Dk, z, y, 0, nullptr) == SSM_OK);
    EXPECT(check_state_update(256, 4096, 16, 1, nullptr, x, dl, A, B, C, Dk, z, y, 0, nullptr) == SSM_EINVAL);
    EXPECT(check_state_update(256, 4096, 16, 1, h, x, dl, A, B, C, Dk, z, x, 0, nullptr) == SSM_EINVAL);
    EXPECT(check_state_update(256, 4096, 16, 1, h, x, dl, A, B, C, Dk, z, y, 2, nullptr) == SSM_EINVAL);
    EXPECT(check_state_update(256, 4096, 257, 1, h, x, dl, A, B, C, Dk, z, y, 0, nullptr) == SSM_EUNSUPPORTED);
    EXPECT(check_state_update(0, 4096, 16, 1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr, nullptr, nullptr, 0, nullptr) == SSM_OK);
    // multi-head SSD scan
    {
        const float *bias = static_cast<const float *>(P(base + 11 * gap));
        auto sdg = [&](int64_t b, int64_t l, int64_t hh, int64_t pd, int64_t n, int64_t g, int dt, const void *y_,
                       const float *hl_) {
            return check_ssd(b, l, hh, pd, n, g, dt, x, dl, A, B, C, Dk, z, bias, h0, hl_, y_, 1);
        };
        auto sd = [&](int64_t b, int64_t l, int64_t hh, int64_t pd, int64_t n, int dt, const void *y_, const float *hl_) {
            return sdg(b, l, hh, pd, n, 1, dt, y_, hl_);
        };
        EXPECT(sd(4, 4096, 64, 64, 128, SSM_DTYPE_BF16, y, hl) == SSM_OK);
        // other head dims, state sizes and fp32 take the generic kernel; more than 256 states no
        EXPECT(sd(4, 4096, 64, 32, 128, SSM_DTYPE_BF16, y, hl) == SSM_OK);
        EXPECT(sd(4, 4096, 64, 64, 16, SSM_DTYPE_BF16, y, hl) == SSM_OK);
        EXPECT(sd(4, 4096, 64, 64, 128, SSM_DTYPE_F32, y, hl) == SSM_OK);
        EXPECT(sd(4, 4096, 64, 64, 257, SSM_DTYPE_BF16, y, hl) == SSM_EUNSUPPORTED);
        EXPECT(sd(4, 4096, 64, 64, 128, 7, y, hl) == SSM_EINVAL);
        EXPECT(sd(-1, 4096, 64, 64, 128, SSM_DTYPE_BF16, y, hl) == SSM_EINVAL);
        EXPECT(sd(4, 4096, 64, 64, 128, SSM_DTYPE_BF16, nullptr, hl) == SSM_EINVAL);
        EXPECT(sd(4, 4096, 64, 64, 128, SSM_DTYPE_BF16, P(base + 16), hl) == SSM_EINVAL);   // overlaps x
        EXPECT(sd(4, 4096, 64, 64, 128, SSM_DTYPE_BF16, y, h0) == SSM_EINVAL);            // h_last on h0
        EXPECT(sd(0, 4096, 64, 64, 128, SSM_DTYPE_BF16, nullptr, nullptr) == SSM_OK);
        EXPECT(check_ssd(4, 16, 64, 64, 128, 1, 1, x, dl, A, B, C, Dk, z, bias, h0, hl, y, 2) == SSM_EINVAL);
        // B/C groups: ngroups >= 1 dividing nheads; on the generic kernel a group's channels
        // must fill whole 64-channel workgroups
        EXPECT(sdg(4, 4096, 64, 64, 128, 8, SSM_DTYPE_BF16, y, hl) == SSM_OK);
        EXPECT(sdg(4, 4096, 64, 64, 128, 64, SSM_DTYPE_BF16, y, hl) == SSM_OK);
        EXPECT(sdg(4, 4096, 64, 64, 128, 0, SSM_DTYPE_BF16, y, hl) == SSM_EINVAL);
        EXPECT(sdg(4, 4096, 64, 64, 128, 3, SSM_DTYPE_BF16, y, hl) == SSM_EINVAL);
        EXPECT(sdg(4, 4096, 64, 32, 128, 32, SSM_DTYPE_BF16, y, hl) == SSM_OK);           // 2 heads x 32
        EXPECT(sdg(4, 4096, 64, 32, 128, 64, SSM_DTYPE_BF16, y, hl) == SSM_EUNSUPPORTED); // 1 head x 32
        EXPECT(sdg(4, 4096, 64, 64, 128, 4, SSM_DTYPE_F32, y, hl) == SSM_OK);
    }
    EXPECT(std::strcmp(ssm_status_str(SSM_EWORKSPACE), "workspace too small") == 0);
    std::printf("%s: %d failure(s)\n", fails ? "FAILED" : "ok", fails);
    return fails ? 1 : 0;
}
