// gemv_cfg.h -- launch configurations of the q4_0 GEMV call sites (host side).
#pragma once

#include "gemv_q4_0.h"

namespace qd {

// GEMV launch configurations: rows per slot, waves, block groups per item,
// register buffers, items per unrolled chunk, non-temporal weight loads (the
// template arguments), a cap on the grid and on the lanes per row.  Chosen
// per call site by timing the step's shapes on MI355X over rotated weight
// copies; the lanes-per-row count follows K.
struct GemvCfg {
    int rps, nw, bg, nbuf, unr, ntl, grid_cap, lpr_max;
};
#define QD_CFG_O 2, 8, 1, 2, 4, false      // o-proj, N ~ hidden
#define QD_CFG_DOWN 2, 8, 1, 3, 6, false   // down, long rows
#define QD_CFG_QKV 3, 8, 1, 2, 4, false    // q|k|v
#define QD_CFG_GU 2, 4, 2, 2, 8, false     // gate|up (16 lanes per row)
#define QD_CFG_HEAD 4, 4, 1, 2, 10, true   // LM head (streamed once)
// one row per slot: for matrices whose row tiles at the sizes above give too
// few workgroups to fill the chip (small models; the same waves, so the x
// staging registers do not grow)
#define QD_CFG_O_S 1, 8, 1, 2, 4, false
#define QD_CFG_DOWN_S 1, 8, 1, 3, 6, false
#define QD_CFG_QKV_S 1, 8, 1, 2, 4, false
static constexpr GemvCfg CFG_O = {QD_CFG_O, 1 << 30, 64};
static constexpr GemvCfg CFG_DOWN = {QD_CFG_DOWN, 1 << 30, 64};
static constexpr GemvCfg CFG_QKV = {QD_CFG_QKV, 1 << 30, 64};
static constexpr GemvCfg CFG_GU = {QD_CFG_GU, 512, 16};
static constexpr GemvCfg CFG_HEAD = {QD_CFG_HEAD, 2048, 64};
static constexpr GemvCfg CFG_O_S = {QD_CFG_O_S, 1 << 30, 64};
static constexpr GemvCfg CFG_DOWN_S = {QD_CFG_DOWN_S, 1 << 30, 64};
static constexpr GemvCfg CFG_QKV_S = {QD_CFG_QKV_S, 1 << 30, 64};
// a call site takes its one-row configuration below this many workgroups
#ifndef QD_GEMV_SMALL_GRID
#define QD_GEMV_SMALL_GRID 128
#endif
static constexpr int GEMV_MAX_LDS = 64 * 1024;

// lanes per row: the largest of 64/32/16/8, at most the configuration's
// limit, dividing the number of blocks
static int pick_lpr(int nb, int lmax = 64)
{
    for (int l = lmax; l >= 8; l >>= 1)
        if (nb % l == 0)
            return l;
    return 8;
}

static int rows_per_tile(const GemvCfg& c, int lpr) { return c.nw * (WAVE / lpr) * c.rps; }

static size_t gemv_lds_bytes(int nb) { return (size_t)gemv_lds_floats(nb) * sizeof(float); }

static int gemv_grid(const GemvCfg& c, int lpr, int N)
{
    const int nt = (N + rows_per_tile(c, lpr) - 1) / rows_per_tile(c, lpr);
    const int g = nt < c.grid_cap ? nt : c.grid_cap;
    return g > 0 ? g : 1;
}

// Launch kernel template KT<LPR, P...> with P = (RPS, NW, BG, NBUF, UNR, NTL).
#define QD_UNPACK(...) __VA_ARGS__
#define QD_NW_(a, b, c, d, e, f) b
#define QD_NW(...) QD_NW_(__VA_ARGS__)
#define QD_GEMV_ONE(KT, L, P, grid, lds, s, ...) \
    hipLaunchKernelGGL((KT<L, QD_UNPACK P>), dim3(grid), dim3(QD_NW P * WAVE), lds, s, __VA_ARGS__)
#define QD_GEMV(KT, P, l, grid, lds, s, ...)                                                      \
    switch (l) {                                                                                   \
    case 64: QD_GEMV_ONE(KT, 64, P, grid, lds, s, __VA_ARGS__); break;                              \
    case 32: QD_GEMV_ONE(KT, 32, P, grid, lds, s, __VA_ARGS__); break;                              \
    case 16: QD_GEMV_ONE(KT, 16, P, grid, lds, s, __VA_ARGS__); break;                              \
    default: QD_GEMV_ONE(KT, 8, P, grid, lds, s, __VA_ARGS__); break;                               \
    }

}  // namespace qd
