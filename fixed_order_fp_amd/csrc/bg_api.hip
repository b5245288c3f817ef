// bg_api.hip -- the C ABI of libbitgemm: descriptor validation, order
// signature, launch plans, and the entry points declared in bitgemm.h.
//
// A descriptor is a frozen record of the fields that decide the arithmetic;
// identical records must produce identical bits ("Taming Bitwise Behavior",
// section 4).  The schedule sub-struct is excluded from the signature: it only
// chooses tiles and waves (section 3.2.2; appendix E).  A descriptor the library
// cannot realise exactly is refused, never replaced by another order (the
// "GPU Mechanism" page's forced-algorithm refusal).
#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "bg_internal.h"

#ifndef BG_PROFILE_HASH
#define BG_PROFILE_HASH 0ull
#endif

namespace {

thread_local std::string g_last_error;

bg_status fail(bg_status s, const std::string& msg)
{
    g_last_error = msg;
    return s;
}

// ---- device check: gfx950 only, cached per device ------------------------
std::mutex g_arch_mu;
std::vector<int> g_arch_ok;  // -1 unknown, 0 no, 1 yes

bg_status check_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(BG_E_HIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(g_arch_mu);
    if ((int)g_arch_ok.size() <= dev) g_arch_ok.resize(dev + 1, -1);
    if (g_arch_ok[dev] < 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(BG_E_HIP, "hipGetDeviceProperties failed");
        g_arch_ok[dev] = std::string(prop.gcnArchName).rfind("gfx950", 0) == 0 ? 1 : 0;
    }
    if (!g_arch_ok[dev]) return fail(BG_E_ARCH, "libbitgemm runs on gfx950 (MI355X) only");
    return BG_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// An AQL dispatch packet holds each grid dimension as a 32-bit count of
// work-items, so a launch of `groups` workgroups of `threads` lanes must keep
// groups * threads below 2^32; shapes past that are refused, never launched.
bool grid_fits(int64_t groups, int64_t threads) { return groups >= 0 && groups <= 0xffffffffLL / threads; }

bool tiles_fit(int64_t M, int64_t N, int bm, int bn, int threads)
{
    const int64_t tm = (M + bm - 1) / bm, tn = (N + bn - 1) / bn;
    return tm <= 0xffffffffLL / threads && tn <= 0xffffffffLL / threads && grid_fits(tm * tn, threads);
}

// ---- order signature: FNV-1a 64 over the order fields, two lanes ----------
struct Fnv {
    uint64_t h[2] = {0xcbf29ce484222325ull, 0x84222325cbf29ce4ull};
    void bytes(const void* p, size_t n)
    {
        const unsigned char* b = (const unsigned char*)p;
        for (size_t i = 0; i < n; i++) {
            h[0] = (h[0] ^ b[i]) * 0x100000001b3ull;
            h[1] = (h[1] ^ (unsigned char)(b[i] + 0x5b)) * 0x100000001b3ull;
        }
    }
    void u32(uint32_t v) { bytes(&v, 4); }
    void i64(int64_t v) { bytes(&v, 8); }
    void u64(uint64_t v) { bytes(&v, 8); }
};

int instruction_k(uint32_t mfma)
{
    switch (mfma) {
    case BG_MFMA_F32_32X32X16_BF16: return 16;
    case BG_MFMA_F32_16X16X32_BF16: return 32;
    case BG_MFMA_I32_32X32X32_I8: return 32;
    case BG_MFMA_I32_16X16X64_I8: return 64;
    default: return 0;
    }
}

// Cut points for K; BG_OK or BG_E_INVALID.
bg_status make_cuts(const bg_gemm_desc* d, int64_t K, int64_t* cuts)
{
    const int S = (int)d->split_k;
    if (S < 1 || S > BG_MAX_SPLIT) return fail(BG_E_INVALID, "split_k must be in 1..64");
    if (K < 1) return fail(BG_E_INVALID, "K must be >= 1");
    if (d->cut_rule == BG_CUT_EXPLICIT) {
        if (d->cuts[0] != 0 || d->cuts[S] != K)
            return fail(BG_E_INVALID, "explicit cuts must start at 0 and end at K");
        for (int s = 0; s < S; s++) {
            if (d->cuts[s] >= d->cuts[s + 1]) return fail(BG_E_INVALID, "explicit cuts must increase");
            cuts[s] = d->cuts[s];
        }
        cuts[S] = K;
        return BG_OK;
    }
    if (d->cut_rule != BG_CUT_UNIT_REMAINDER_LAST) return fail(BG_E_INVALID, "unknown cut_rule");
    if (d->cut_unit < 1) return fail(BG_E_INVALID, "cut_unit must be >= 1");
    cuts[0] = 0;
    if (S == 1) {
        cuts[1] = K;
        return BG_OK;
    }
    const int64_t unit = d->cut_unit;
    const int64_t span = (K / (unit * S)) * unit;
    if (span <= 0) return fail(BG_E_INVALID, "a split would be empty: K < unit * split_k");
    for (int s = 1; s < S; s++) cuts[s] = (int64_t)s * span;
    cuts[S] = K;
    return BG_OK;
}

// Field checks shared by the GEMM entry points.
bg_status check_common_order(const bg_gemm_desc* d)
{
    if (!d) return fail(BG_E_INVALID, "descriptor is NULL");
    if (d->version != 1) return fail(BG_E_INVALID, "descriptor version must be 1");
    if (d->k_order != BG_K_ASCENDING) return fail(BG_E_INVALID, "unknown k_order");
    if (d->short_turn == BG_SHORT_TURN_FIRST)
        return fail(BG_E_UNSUPPORTED, "short_turn FIRST is not built: a short turn runs last");
    if (d->short_turn != BG_SHORT_TURN_LAST) return fail(BG_E_INVALID, "unknown short_turn");
    if (d->k_slot_layout == BG_SLOTS_STRIDED)
        return fail(BG_E_UNSUPPORTED, "strided k slots are not built");
    if (d->k_slot_layout != BG_SLOTS_CONTIGUOUS) return fail(BG_E_INVALID, "unknown k_slot_layout");
    if (d->acc_update == BG_ACC_SEPARATE_ADD)
        return fail(BG_E_UNSUPPORTED, "acc_update SEPARATE_ADD is not built");
    if (d->acc_update != BG_ACC_IN_MFMA) return fail(BG_E_INVALID, "unknown acc_update");
    if (d->odd_rule != BG_ODD_CARRY_LAST) return fail(BG_E_INVALID, "unknown odd_rule");
    if (d->rounding_point != BG_ROUND_AFTER_COMBINE_RNE) return fail(BG_E_INVALID, "unknown rounding_point");
    if (d->mfma_profile_hash != BG_PROFILE_HASH)
        return fail(BG_E_PROFILE, "descriptor's MFMA profile hash is not the one this library was built for");
    return BG_OK;
}

// Speed only: a tile shape for the problem (every shape gives the same bits).
// Chosen from measurements on MI355X: large outputs take the pipelined
// 320x256 / 256x320 tiles (8 waves, two rounds of workgroups at the headline
// size); smaller outputs take smaller pipelined tiles with deeper LDS
// pipelines, since each workgroup's walk over K is then bound by copy
// latency rather than by the MFMA rate.  Needs p.S and p.cuts set.
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device, for the tile choices (speed only; 256
// on MI355X, and 256 when no device can be asked, as in a host-only plan
// query).  Read once per device.
std::mutex g_cu_mu;
std::vector<int> g_cus;
int64_t device_cus()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    std::lock_guard<std::mutex> lk(g_cu_mu);
    if ((int)g_cus.size() <= dev) g_cus.resize(dev + 1, 0);
    if (!g_cus[dev]) {
        int n = 0;
        g_cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0
                         ? n
                         : 256;
    }
    return g_cus[dev];
}

// Speed only (int32 sums are exact in any order): the pipelined int8 tile.
// Outputs of at least 1.5 rounds of 256x256 tiles take that tile (the fewest
// operand bytes per product; 1.27x the 128x128 tile's rate on the stacked
// 16000 x 38912 x 2560 product).  Below that, where 128x128 tiles give a
// workgroup per CU, the big tile is the one that moves fewer operand bytes
// per CU: rounds x workgroups per CU x (BM + BN), one workgroup per CU
// (128x192, 8 waves) costing ~1.4x per byte against two (128x128, 5 stages),
// as measured at 1024 x 6144 x 2048 with inputs not in the MALL.  Otherwise
// deep-pipelined small tiles.  The large and mid-size tiles take 128-byte k
// tiles in two stages (whole 128-byte lines per copy: 3-13 % faster than
// the 64-byte rings on these shapes, measured on MI355X) where the copy
// offsets fit, else the 64-byte ring.
void choose_w8a8_pipe(bg::W8A8Plan& p, int64_t M, int64_t N, int64_t lda, int64_t ldw)
{
    const int64_t n_cu = device_cus();
    const int64_t t128 = ceil_div(M, 128) * ceil_div(N, 128), t192 = ceil_div(M, 128) * ceil_div(N, 192);
    p.path = 2;
    if (ceil_div(M, 256) * ceil_div(N, 256) >= n_cu * 3 / 2) {
        p.bm = 256, p.bn = 256, p.waves_m = 2, p.waves_n = 4;
        p.stages = bg::i8_offsets_fit(256, 256, lda, ldw) ? 2 : 4;
    } else if (t128 >= 192) {
        const double c128 = (double)ceil_div(t128, 2 * n_cu) * 2 * 256;
        const double c192 = (double)ceil_div(t192, n_cu) * 320 * 1.4;
        if (c192 < c128) {
            // 128-byte k tiles in a ring of three (two in flight, full
            // pointers, no offset limit): 4 % faster than two stages on
            // inputs streamed from HBM
            p.bm = 128, p.bn = 192, p.waves_m = 4, p.waves_n = 2, p.stages = 3;
        } else {
            p.bm = 128, p.bn = 128, p.waves_m = 2, p.waves_n = 2;
            p.stages = bg::i8_offsets_fit(p.bm, p.bn, lda, ldw) ? 2 : 5;
        }
    } else {
        p.bm = 64, p.bn = 64, p.waves_m = 2, p.waves_n = 2, p.stages = 8;
    }
}

// ---- tiles for split-K ---------------------------------------------------
// Time of one pipelined workgroup over `turns` k tiles of 32, in us: a
// per-turn cost measured on MI355X for each tile (the deep split of a
// 256 x 2560 x 9728 product, one workgroup per CU, at the clock these kernels
// settle at; the 8-wave 256 x 256 tile measured ahead of the 4-wave one once
// every CU is busy), plus 0.5 us, one turn per stage for the pipeline fill,
// and the fp32 partial tile's store at 30 GB/s per CU.  Workgroups that share
// a CU (as many as its LDS holds, while there are more workgroups than CUs)
// each run that much slower.  The constants were fitted to the split sweep of
// that product (S = 2 .. 16, the tiles and pairs below); the model ranks
// tiles, it does not predict times.
// The 64-deep tiles' per-turn costs (per 32 of k) come from the same sweep
// where it was measured (64x64, 128x64, 128x128 at S = 1, 2, 4) and are
// scaled from the 32-deep ones by the measured ratio elsewhere (0.87).
struct PipeTileCost {
    int bm, bn, bk, wm, wn, ns;
    double turn_us;
};
const PipeTileCost kPipeCosts[] = {
    {256, 256, 32, 2, 4, 4, 0.858}, {256, 256, 32, 2, 2, 4, 0.900}, {192, 256, 32, 2, 4, 4, 0.613},
    {256, 128, 32, 2, 2, 4, 0.510}, {192, 128, 32, 2, 2, 4, 0.407}, {128, 128, 32, 2, 2, 4, 0.333},
    {128, 128, 32, 2, 2, 8, 0.327}, {128, 64, 32, 2, 2, 4, 0.293},  {128, 64, 32, 2, 2, 8, 0.259},
    {64, 128, 32, 2, 2, 4, 0.293},  {64, 128, 32, 2, 2, 8, 0.267},  {64, 64, 32, 2, 2, 8, 0.189},
    {128, 64, 32, 4, 2, 8, 0.259},  {64, 128, 32, 2, 4, 8, 0.267},  {256, 256, 64, 2, 4, 2, 0.750},
    {192, 128, 64, 2, 2, 4, 0.354}, {128, 128, 64, 2, 2, 4, 0.319}, {128, 64, 64, 2, 2, 4, 0.220},
    {128, 64, 64, 4, 2, 4, 0.220},  {64, 64, 64, 2, 2, 6, 0.148}};

const PipeTileCost* pipe_cost(int bm, int bn, int bk, int wm, int wn, int ns)
{
    for (const PipeTileCost& c : kPipeCosts)
        if (c.bm == bm && c.bn == bn && c.bk == bk && c.wm == wm && c.wn == wn && c.ns == ns) return &c;
    return nullptr;
}

double wg_us(const PipeTileCost& c, int64_t turns)
{
    return 0.5 + (double)(turns + c.ns) * c.turn_us + (double)c.bm * c.bn * 4.0 / 30e3;
}

int pipe_lds_bytes(const PipeTileCost& c) { return c.ns * (c.bm + c.bn) * c.bk * 2; }

// Longest-first list schedule of two kinds of workgroups on n_cu slots, one
// at a time per slot: the longer kind is dealt out first (some slots take
// one more of them), then each shorter workgroup goes to the slot that frees
// up first.  Returns the time the last slot finishes.
double lpt_slots(int64_t na, double ta, int64_t nb, double tb, int64_t n_cu)
{
    if (tb > ta) std::swap(na, nb), std::swap(ta, tb);
    const int64_t q = na / n_cu, r = na % n_cu;
    const double lo = (double)q * ta, hi = (double)(q + (r ? 1 : 0)) * ta;
    if (nb <= 0) return hi;
    if (tb <= 0.0) return hi;
    // the earliest time T by which the CUs at `lo` (n_cu - r of them) and at
    // `hi` (r) have room for nb shorter workgroups
    auto fits = [&](double T) {
        const int64_t a = T >= lo ? (int64_t)((T - lo) / tb + 1e-9) : 0;
        const int64_t b = T >= hi ? (int64_t)((T - hi) / tb + 1e-9) : 0;
        return (n_cu - r) * a + r * b >= nb;
    };
    // fits() grows with T, and a CU's load changes only at lo + k tb or
    // hi + k tb: the answer is the first of either family that fits
    auto first_k = [&](double base) {  // smallest k >= 1 with fits(base + k tb), by bisection
        int64_t a = 1, b = nb + 1;         // fits(base + (nb + 1) tb) always holds
        while (a < b) {
            const int64_t m = a + (b - a) / 2;
            if (fits(base + (double)m * tb)) b = m;
            else a = m + 1;
        }
        return a;
    };
    return std::min(std::max(lo + (double)first_k(lo) * tb, hi), hi + (double)first_k(hi) * tb);
}

// lpt_slots with `lds` bytes per workgroup: a CU holds 160 KiB / lds of
// them, and while there are more workgroups than CUs it runs up to that many
// at once, each proportionally slower
double lpt2(int64_t na, double ta, int64_t nb, double tb, int64_t n_cu, int lds)
{
    const double per_cu = std::max(1, (160 * 1024) / std::max(lds, 1));
    const double share = std::min(per_cu, std::max(1.0, (double)(na + nb) / (double)n_cu));
    return lpt_slots(na, ta * share, nb, tb * share, (int64_t)((double)n_cu * share));
}

struct DualPair {
    int bk, bm, bn, wm, wn, ns, bm2, bn2, wm2, wn2, ns2;
};
// must list exactly the pairs bg_gemm_bf16.hip compiles in; on a tie of the
// model below the earlier pair wins (128x128 + 128x64 on 64-deep tiles
// measured 6 % ahead of 128x128 + 64x64 at S = 8, which the model ties)
const DualPair kDualPairs[] = {{32, 256, 256, 2, 2, 4, 64, 64, 2, 2, 8}, {32, 256, 256, 2, 2, 4, 128, 64, 2, 2, 4},
                               {32, 256, 128, 2, 2, 4, 64, 64, 2, 2, 8}, {32, 192, 128, 2, 2, 4, 64, 64, 2, 2, 8},
                               {32, 128, 128, 2, 2, 4, 64, 64, 2, 2, 8}, {32, 256, 256, 2, 4, 4, 128, 64, 4, 2, 8},
                               {32, 256, 256, 2, 4, 4, 64, 128, 2, 4, 8}, {64, 256, 256, 2, 4, 2, 128, 64, 4, 2, 4},
                               {64, 128, 128, 2, 2, 4, 128, 64, 2, 2, 4}, {64, 128, 128, 2, 2, 4, 64, 64, 2, 2, 6}};

// The split grid's tiles (S > 1): every single tile of the cost table and
// every compiled (other splits, last split) pair is scored by lpt2 over the
// splits' depths; the cheapest wins, a single tile on a tie.
void choose_split_tiles(bg::GemmPlan& p, int64_t M, int64_t N, int64_t lda, int64_t ldb)
{
    const int64_t n_cu = device_cus();
    int64_t body = 0;
    for (int s = 0; s + 1 < p.S; s++) body = std::max<int64_t>(body, p.cuts.c[s + 1] - p.cuts.c[s]);
    const int64_t last = p.cuts.c[p.S] - p.cuts.c[p.S - 1];
    const int64_t tb = (body + 31) / 32, tl = (last + 31) / 32;
    auto tiles = [&](int bm, int bn) { return ceil_div(M, bm) * ceil_div(N, bn); };
    double best = 0.0;
    bool have = false;
    for (const PipeTileCost& c : kPipeCosts) {
        if (c.bm > 64 && M <= 64) continue;
        // some costed shapes exist only as the last split's half of a pair
        if (!bg::gemm_bf16_has_tile(BG_MFMA_F32_32X32X16_BF16, c.bm, c.bn, c.bk, c.wm, c.wn, 2, c.ns)) continue;
        if (c.ns == 2 && !bg::pipe_offsets_fit(c.bm, c.bn, lda, ldb)) continue;
        const int64_t n = tiles(c.bm, c.bn);
        const double t = lpt2(n * (p.S - 1), wg_us(c, tb), n, wg_us(c, tl), n_cu, pipe_lds_bytes(c));
        if (!have || t < best) {
            have = true, best = t;
            p.bm = c.bm, p.bn = c.bn, p.bk = c.bk, p.waves_m = c.wm, p.waves_n = c.wn, p.direct = 2, p.stages = c.ns;
            p.bm2 = 0, p.bn2 = 0, p.waves_m2 = 0, p.waves_n2 = 0, p.stages2 = 0;
        }
    }
    for (const DualPair& d : kDualPairs) {
        const PipeTileCost* a = pipe_cost(d.bm, d.bn, d.bk, d.wm, d.wn, d.ns);
        const PipeTileCost* b = pipe_cost(d.bm2, d.bn2, d.bk, d.wm2, d.wn2, d.ns2);
        if (!a || !b ||
            !bg::gemm_bf16_has_dual_tile(d.bm, d.bn, d.bk, d.wm, d.wn, d.ns, d.bm2, d.bn2, d.wm2, d.wn2, d.ns2))
            continue;
        if ((d.ns == 2 && !bg::pipe_offsets_fit(d.bm, d.bn, lda, ldb)) ||
            (d.ns2 == 2 && !bg::pipe_offsets_fit(d.bm2, d.bn2, lda, ldb)))
            continue;
        const double ta = wg_us(*a, tb), tl2 = wg_us(*b, tl);
        const double t = lpt2(tiles(d.bm, d.bn) * (p.S - 1), ta, tiles(d.bm2, d.bn2), tl2, n_cu,
                              std::max(pipe_lds_bytes(*a), pipe_lds_bytes(*b)));
        if (t < best) {
            best = t;
            p.bm = d.bm, p.bn = d.bn, p.bk = d.bk, p.waves_m = d.wm, p.waves_n = d.wn, p.direct = 2, p.stages = d.ns;
            p.bm2 = d.bm2, p.bn2 = d.bn2, p.waves_m2 = d.wm2, p.waves_n2 = d.wn2, p.stages2 = d.ns2;
            p.last_first = tl2 >= ta;
        }
    }
}

// whether the last split's workgroups go first (the longer kind first)
bool dual_last_first(const bg::GemmPlan& p)
{
    const PipeTileCost* a = pipe_cost(p.bm, p.bn, p.bk, p.waves_m, p.waves_n, p.stages);
    const PipeTileCost* b = pipe_cost(p.bm2, p.bn2, p.bk, p.waves_m2, p.waves_n2, p.stages2);
    if (!a || !b) return true;
    int64_t body = 0;
    for (int s = 0; s + 1 < p.S; s++) body = std::max<int64_t>(body, p.cuts.c[s + 1] - p.cuts.c[s]);
    const int64_t last = p.cuts.c[p.S] - p.cuts.c[p.S - 1];
    return wg_us(*b, (last + 31) / 32) >= wg_us(*a, (body + 31) / 32);
}

void choose_gemm_tile(bg::GemmPlan& p, int64_t M, int64_t N, int64_t lda, int64_t ldb)
{
    auto set = [&](int bm, int bn, int bk, int wm, int wn, int direct, int stages) {
        p.bm = bm, p.bn = bn, p.bk = bk, p.waves_m = wm, p.waves_n = wn, p.direct = direct, p.stages = stages;
    };
    if (p.mfma != BG_MFMA_F32_32X32X16_BF16) {
        if (M > 32 && N >= 128 && M >= 128) set(128, 128, 64, 2, 2, 0, 0);
        else if (M > 16) set(64, 64, 64, 2, 2, 0, 0);
        else set(32, 32, 64, 1, 1, 0, 0);
        return;
    }
    const int64_t n_cu = device_cus();
    // fraction of the last round of workgroups that is busy, weighted in
    auto quant = [&](int64_t bm, int64_t bn, int per_cu) {
        const int64_t wgs = ceil_div(M, bm) * ceil_div(N, bn) * p.S;
        const int64_t slots = n_cu * per_cu;
        return (double)(M * N) / (double)(ceil_div(wgs, slots) * slots * bm * bn) * p.S;
    };
    if (ceil_div(M, 256) * ceil_div(N, 256) * p.S >= n_cu * 3 / 2) {
        // 64-deep k tiles in two stages (whole 128-byte lines per copy) where
        // the copy offsets fit, else the 32-deep four-stage ring
        const bool tall = quant(320, 256, 1) >= quant(256, 320, 1);
        const bool deep = bg::pipe_offsets_fit(tall ? 320 : 256, tall ? 256 : 320, lda, ldb);
        if (tall) deep ? set(320, 256, 64, 2, 4, 2, 2) : set(320, 256, 32, 2, 4, 2, 4);
        else deep ? set(256, 320, 64, 4, 2, 2, 2) : set(256, 320, 32, 4, 2, 2, 4);
        return;
    }
    // small M: each CU streams its strip of W from HBM; 64-deep k tiles
    // (whole 128-byte lines per copy) in a ring of six stages
    if (M <= 32) {  // 304 workgroups of 32x64 stream W faster than 152 of 64x64
        set(32, 64, 64, 1, 2, 2, 6);
        return;
    }
    if (M <= 64) {
        set(64, 64, 64, 2, 2, 2, 6);
        return;
    }
    if (p.S > 1) {
        // a remainder split at least twice as deep as the others: score the
        // pairs of tiles too (the longest-first model below); otherwise the
        // splits are about even and the copy-time model below picks one tile
        int64_t body = 0;
        for (int s = 0; s + 1 < p.S; s++) body = std::max<int64_t>(body, p.cuts.c[s + 1] - p.cuts.c[s]);
        if (p.cuts.c[p.S] - p.cuts.c[p.S - 1] >= 2 * body) {
            choose_split_tiles(p, M, N, lda, ldb);
            return;
        }
    }
    // deep splits: the tile whose busiest CU finishes first.  Each CU moves
    // operands at ~38 GB/s with 32-deep k tiles (64-byte row pieces) and
    // ~50 GB/s with 64-deep ones (whole 128-byte lines), and multiplies at
    // ~8.1 TFLOP/s (all measured on these kernels, at the clock they settle
    // at), so a tile costs rounds of workgroups x max(copy time, MFMA time)
    // of one workgroup over the deepest split.  Shallow splits: small tiles
    // (their prologue and epilogue weigh less).
    auto wgs = [&](int64_t bm, int64_t bn) { return ceil_div(M, bm) * ceil_div(N, bn) * p.S; };
    const int64_t turns = p.cuts.c[1] / 32;
    if (turns >= 64) {
        struct Cand { int bm, bn, bk, wm, wn, ns; };
        static const Cand cands[] = {{320, 256, 32, 2, 4, 4}, {256, 256, 32, 2, 4, 4}, {192, 256, 32, 2, 4, 4},
                                     {256, 128, 32, 2, 2, 4}, {192, 128, 32, 2, 2, 4}, {128, 128, 32, 2, 2, 5},
                                     {128, 64, 32, 2, 2, 8},  {64, 64, 32, 2, 2, 8},   {192, 128, 64, 2, 2, 4},
                                     {128, 128, 64, 2, 2, 4}, {128, 64, 64, 2, 2, 4},  {64, 64, 64, 2, 2, 6}};
        int64_t kmax = 0;
        for (int s = 0; s < p.S; s++) kmax = std::max<int64_t>(kmax, p.cuts.c[s + 1] - p.cuts.c[s]);
        const Cand* pick = nullptr;
        double best = 0.0;
        for (const Cand& c : cands) {
            const double copy = (double)(c.bm + c.bn) * (double)kmax * 2.0 / (c.bk == 64 ? 50e9 : 38e9);
            const double mfma = (double)c.bm * c.bn * (double)kmax * 2.0 / 8.1e12;
            const double t = (double)ceil_div(wgs(c.bm, c.bn), n_cu) * std::max(copy, mfma);
            if (!pick || t < best) pick = &c, best = t;
        }
        set(pick->bm, pick->bn, pick->bk, pick->wm, pick->wn, 2, pick->ns);
        return;
    }
    if (wgs(64, 64) <= 2048) set(64, 64, 32, 2, 2, 2, 8);
    else set(128, 64, 32, 2, 2, 2, 4);
}

// the reduction descriptor of a GEMM with fused reductions: fp32 values (C)
bg_status check_fused_reduce(const bg_reduce_desc* rd)
{
    if (!rd) return fail(BG_E_INVALID, "NULL reduction descriptor");
    if (rd->version != 1) return fail(BG_E_INVALID, "reduction descriptor version must be 1");
    if (rd->in_type != BG_FP32) return fail(BG_E_INVALID, "the fused reductions read the fp32 C: in_type fp32");
    if (rd->acc_type != BG_FP32 || rd->out_type != BG_FP32) return fail(BG_E_INVALID, "accumulation and output are fp32");
    if (rd->op < BG_RED_SUM || rd->op > BG_RED_SUM_AND_SUMSQ) return fail(BG_E_INVALID, "unknown op");
    if (rd->axis != BG_AXIS_ROW && rd->axis != BG_AXIS_COL) return fail(BG_E_INVALID, "unknown axis");
    if (rd->leaf_order != BG_LEAF_SEQUENTIAL_NO_SEED) return fail(BG_E_INVALID, "unknown leaf_order");
    if (rd->sq_fma != BG_SQ_FUSED && rd->sq_fma != BG_SQ_UNFUSED) return fail(BG_E_INVALID, "unknown sq_fma");
    if (rd->tree != BG_TREE_BALANCED) return fail(BG_E_INVALID, "unknown tree");
    if (rd->odd_rule != BG_ODD_CARRY_LAST) return fail(BG_E_INVALID, "unknown odd_rule");
    if (rd->leaf_len != 32) return fail(BG_E_UNSUPPORTED, "only leaves of 32 elements are built");
    return BG_OK;
}

// leaves and outputs of the fused reduction; workspace bytes
void fused_reduce_shape(const bg_reduce_desc* rd, int64_t M, int64_t N, int64_t& n_leaf, int64_t& n_out,
                        size_t& bytes)
{
    n_out = rd->axis == BG_AXIS_COL ? N : M;
    const int64_t len = rd->axis == BG_AXIS_COL ? M : N;
    n_leaf = (len + 31) / 32;
    const int arrays = ((rd->op & BG_RED_SUM) ? 1 : 0) + ((rd->op & BG_RED_SUMSQ) ? 1 : 0);
    bytes = (size_t)n_leaf * (size_t)n_out * sizeof(float) * (size_t)arrays;
}

// ---- the static scratch of bg_gemm_bf16_noalloc -----------------------------
// Split-K partials of the allocation-free entry point live here: one copy per
// GPU, allocated with the library's code object when it is loaded on that GPU
// and held until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: its device address is taken once per
// device with hipGetSymbolAddress (that device current) and only that address
// is handed to kernels.
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device; nullptr until taken

bg_status scratch_for_current_device(void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(BG_E_HIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(BG_E_HIP, std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return BG_OK;
}

}  // namespace

namespace bg {
// the descriptor JSON reader and writer report their refusals here
bg_status json_fail(bg_status s, const std::string& msg) { return fail(s, msg); }
}  // namespace bg

extern "C" {

int bg_abi_version(void) { return BG_ABI_VERSION; }

uint64_t bg_profile_hash(void) { return BG_PROFILE_HASH; }

const char* bg_last_error(void) { return g_last_error.c_str(); }

const char* bg_status_str(bg_status s)
{
    switch (s) {
    case BG_OK: return "ok";
    case BG_E_INVALID: return "invalid argument";
    case BG_E_UNSUPPORTED: return "unsupported descriptor";
    case BG_E_WORKSPACE: return "workspace missing or too small";
    case BG_E_ALIGN: return "misaligned pointer or leading dimension";
    case BG_E_ARCH: return "device is not gfx950";
    case BG_E_PROFILE: return "MFMA profile mismatch";
    case BG_E_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

bg_status bg_desc_default_gemm(bg_gemm_desc* d)
{
    if (!d) return fail(BG_E_INVALID, "descriptor is NULL");
    *d = bg_gemm_desc{};
    d->version = 1;
    d->a_type = BG_BF16;
    d->b_type = BG_BF16;
    d->acc_type = BG_FP32;
    d->out_type = BG_BF16;
    d->mfma = BG_MFMA_F32_32X32X16_BF16;
    d->acc_update = BG_ACC_IN_MFMA;
    d->k_order = BG_K_ASCENDING;
    d->short_turn = BG_SHORT_TURN_LAST;
    d->k_slot_layout = BG_SLOTS_CONTIGUOUS;
    d->split_k = 1;
    d->cut_rule = BG_CUT_UNIT_REMAINDER_LAST;
    d->cut_unit = 256;
    d->partial_type = BG_FP32;
    d->merge_type = BG_FP32;
    d->combine = BG_COMBINE_BALANCED;
    d->odd_rule = BG_ODD_CARRY_LAST;
    d->rounding_point = BG_ROUND_AFTER_COMBINE_RNE;
    d->epilogue = BG_EPI_NONE;
    d->mfma_profile_hash = BG_PROFILE_HASH;
    return BG_OK;
}

bg_status bg_desc_default_reduce(bg_reduce_desc* d)
{
    if (!d) return fail(BG_E_INVALID, "descriptor is NULL");
    *d = bg_reduce_desc{};
    d->version = 1;
    d->in_type = BG_FP32;
    d->acc_type = BG_FP32;
    d->op = BG_RED_SUM_AND_SUMSQ;
    d->axis = BG_AXIS_ROW;
    d->leaf_len = 32;
    d->leaf_order = BG_LEAF_SEQUENTIAL_NO_SEED;
    d->sq_fma = BG_SQ_FUSED;
    d->tree = BG_TREE_BALANCED;
    d->odd_rule = BG_ODD_CARRY_LAST;
    d->out_type = BG_FP32;
    return BG_OK;
}

bg_status bg_desc_signature(const bg_gemm_desc* d, uint64_t sig[2])
{
    if (!d || !sig) return fail(BG_E_INVALID, "NULL argument");
    Fnv f;
    f.u32(d->version);
    f.u32(d->a_type);
    f.u32(d->b_type);
    f.u32(d->acc_type);
    f.u32(d->out_type);
    f.u32(d->mfma);
    f.u32(d->acc_update);
    f.u32(d->k_order);
    f.u32(d->short_turn);
    f.u32(d->k_slot_layout);
    f.u32(d->split_k);
    f.u32(d->cut_rule);
    if (d->cut_rule == BG_CUT_EXPLICIT) {
        const uint32_t S = d->split_k <= BG_MAX_SPLIT ? d->split_k : BG_MAX_SPLIT;
        for (uint32_t s = 0; s <= S; s++) f.i64(d->cuts[s]);
    } else {
        f.u32(d->cut_unit);
    }
    f.u32(d->partial_type);
    f.u32(d->merge_type);
    f.u32(d->combine);
    f.u32(d->odd_rule);
    f.u32(d->rounding_point);
    f.u32(d->epilogue);
    f.u64(d->mfma_profile_hash);
    sig[0] = f.h[0];
    sig[1] = f.h[1];
    return BG_OK;
}

bg_status bg_reduce_desc_signature(const bg_reduce_desc* d, uint64_t sig[2])
{
    if (!d || !sig) return fail(BG_E_INVALID, "NULL argument");
    Fnv f;
    f.u32(0x52454455u);  // a tag so that no reduce signature equals a gemm one
    f.u32(d->version);
    f.u32(d->in_type);
    f.u32(d->acc_type);
    f.u32(d->op);
    f.u32(d->axis);
    f.u32(d->leaf_len);
    f.u32(d->leaf_order);
    f.u32(d->sq_fma);
    f.u32(d->tree);
    f.u32(d->odd_rule);
    f.u32(d->out_type);
    sig[0] = f.h[0];
    sig[1] = f.h[1];
    return BG_OK;
}

bg_status bg_gemm_split_cuts(const bg_gemm_desc* d, int64_t K, int64_t* cuts)
{
    if (!d || !cuts) return fail(BG_E_INVALID, "NULL argument");
    return make_cuts(d, K, cuts);
}

bg_status bg_gemm_workspace_bytes(const bg_gemm_desc* d, int64_t M, int64_t N, int64_t K, size_t* bytes)
{
    (void)K;
    if (!d || !bytes) return fail(BG_E_INVALID, "NULL argument");
    if (M < 0 || N < 0) return fail(BG_E_INVALID, "negative size");
    if (d->split_k < 1 || d->split_k > BG_MAX_SPLIT) return fail(BG_E_INVALID, "split_k must be in 1..64");
    if (N > 0 && M > (INT64_MAX / 256) / N) return fail(BG_E_UNSUPPORTED, "M x N too large");
    *bytes = d->split_k > 1 ? (size_t)d->split_k * (size_t)M * (size_t)N * sizeof(float) : 0;
    return BG_OK;
}

}  // extern "C"

namespace {
// bg_gemm_bf16's descriptor and size checks and its cut points (plan p: S
// and cuts set); nothing here reads memory or the device
bg_status check_gemm_bf16(const bg_gemm_desc* d, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                          int64_t ldc, bg::GemmPlan& p)
{
    bg_status st = check_common_order(d);
    if (st != BG_OK) return st;
    if (d->a_type != BG_BF16 || d->b_type != BG_BF16)
        return fail(BG_E_INVALID, "bg_gemm_bf16 takes bf16 operands");
    if (d->acc_type != BG_FP32) return fail(BG_E_INVALID, "bf16 GEMM accumulates in fp32");
    if (d->out_type != BG_FP32 && d->out_type != BG_BF16) return fail(BG_E_INVALID, "out_type must be fp32 or bf16");
    if (d->mfma != BG_MFMA_F32_32X32X16_BF16 && d->mfma != BG_MFMA_F32_16X16X32_BF16)
        return fail(BG_E_INVALID, "mfma must be a bf16 instruction");
    if (d->partial_type != BG_FP32 || d->merge_type != BG_FP32)
        return fail(BG_E_UNSUPPORTED, "only fp32 partials merged in fp32 are built");
    if (d->combine == BG_COMBINE_SEQUENTIAL) return fail(BG_E_UNSUPPORTED, "sequential combine is not built");
    if (d->combine != BG_COMBINE_BALANCED) return fail(BG_E_INVALID, "unknown combine");
    if (d->epilogue != BG_EPI_NONE) return fail(BG_E_INVALID, "bg_gemm_bf16 has no epilogue");
    if (M < 0 || N < 0) return fail(BG_E_INVALID, "negative size");
    if (lda < K || ldb < K || ldc < N) return fail(BG_E_INVALID, "leading dimension smaller than the row");
    p = bg::GemmPlan{};
    p.S = (int)d->split_k;
    st = make_cuts(d, K, p.cuts.c);
    if (st != BG_OK) return st;
    for (int s = 0; s <= p.S; s++)
        if (p.cuts.c[s] % 8) return fail(BG_E_UNSUPPORTED, "cut points must be multiples of 8");
    p.mfma = (int)d->mfma;
    p.out_bf16 = d->out_type == BG_BF16;
    return BG_OK;
}

// the tiles of plan p (M, N > 0): the descriptor's schedule, or the
// library's choice for the shape
bg_status resolve_gemm_schedule(const bg_gemm_desc* d, int64_t M, int64_t N, int64_t lda, int64_t ldb,
                                bg::GemmPlan& p)
{
    const bg_gemm_schedule& s = d->sched;
    p.group_m = s.group_m;
    if (s.bm || s.bn || s.bk || s.waves_m || s.waves_n) {
        // a pair's other-splits tile need not be compiled on its own (the
        // pair is checked below)
        const bool pair = s.last_bm || s.last_bn || s.last_waves_m || s.last_waves_n || s.last_stages;
        if (!pair && !bg::gemm_bf16_has_tile(p.mfma, s.bm, s.bn, s.bk, s.waves_m, s.waves_n, s.load_path, s.stages))
            return fail(BG_E_UNSUPPORTED, "schedule (bm, bn, bk, waves, load_path, stages) is not compiled in");
        // the two-stage 64-deep tiles (the first compiled entry of their
        // shapes, so also stages 0) address their copies by 32-bit offsets
        auto two_stage = [&](int bm, int bn, int wm, int wn, int ns) {
            return s.load_path == 2 && s.bk == 64 &&
                   (ns == 2 || (ns == 0 && bg::gemm_bf16_has_tile(p.mfma, bm, bn, 64, wm, wn, 2, 2)));
        };
        if (!pair && two_stage(s.bm, s.bn, s.waves_m, s.waves_n, s.stages) &&
            !bg::pipe_offsets_fit(s.bm, s.bn, lda, ldb))
            return fail(BG_E_UNSUPPORTED, "a 64-deep two-stage tile addresses its copies by 32-bit offsets: "
                                          "(bm - 1) x lda and (bn - 1) x ldb must stay below 2^31 elements");
        p.bm = s.bm, p.bn = s.bn, p.bk = s.bk, p.waves_m = s.waves_m, p.waves_n = s.waves_n;
        p.direct = s.load_path;
        p.stages = s.stages;
        if (s.last_bm || s.last_bn || s.last_waves_m || s.last_waves_n || s.last_stages) {
            if (p.S < 2) return fail(BG_E_UNSUPPORTED, "a last-split tile needs split_k > 1");
            if (s.load_path != 2 || p.mfma != BG_MFMA_F32_32X32X16_BF16 ||
                !bg::gemm_bf16_has_dual_tile(s.bm, s.bn, s.bk, s.waves_m, s.waves_n, s.stages, s.last_bm, s.last_bn,
                                             s.last_waves_m, s.last_waves_n, s.last_stages))
                return fail(BG_E_UNSUPPORTED, "the (tile, last-split tile) pair is not compiled in");
            p.bm2 = s.last_bm, p.bn2 = s.last_bn, p.waves_m2 = s.last_waves_m, p.waves_n2 = s.last_waves_n;
            p.stages2 = s.last_stages;
            for (const DualPair& dp : kDualPairs)  // the pair's compiled stage counts where left 0
                if (dp.bk == p.bk && dp.bm == p.bm && dp.bn == p.bn && dp.wm == p.waves_m && dp.wn == p.waves_n &&
                    (!p.stages || dp.ns == p.stages) && dp.bm2 == p.bm2 && dp.bn2 == p.bn2 && dp.wm2 == p.waves_m2 &&
                    dp.wn2 == p.waves_n2 && (!p.stages2 || dp.ns2 == p.stages2)) {
                    p.stages = dp.ns, p.stages2 = dp.ns2;
                    break;
                }
            if (p.bk == 64 && ((p.stages == 2 && !bg::pipe_offsets_fit(p.bm, p.bn, lda, ldb)) ||
                               (p.stages2 == 2 && !bg::pipe_offsets_fit(p.bm2, p.bn2, lda, ldb))))
                return fail(BG_E_UNSUPPORTED, "a 64-deep two-stage tile addresses its copies by 32-bit offsets: "
                                              "(bm - 1) x lda and (bn - 1) x ldb must stay below 2^31 elements");
            p.last_first = dual_last_first(p);
        }
    } else {
        if (s.last_bm || s.last_bn || s.last_waves_m || s.last_waves_n || s.last_stages)
            return fail(BG_E_UNSUPPORTED, "a last-split tile needs the other splits' tile (bm .. waves_n) set");
        choose_gemm_tile(p, M, N, lda, ldb);
    }
    if (!tiles_fit(M, N, p.bm, p.bn, 64 * p.waves_m * p.waves_n) || (p.S > 1 && !grid_fits((M * N + 255) / 256, 256)))
        return fail(BG_E_UNSUPPORTED, "M x N too large for one launch");
    return BG_OK;
}
}  // namespace

extern "C" {

bg_status bg_gemm_bf16_plan(const bg_gemm_desc* d, int64_t M, int64_t N, int64_t K, bg_gemm_schedule* out)
{
    if (!d || !out) return fail(BG_E_INVALID, "NULL argument");
    bg::GemmPlan p{};
    bg_status st = check_gemm_bf16(d, M, N, K, K, K, N, p);
    if (st != BG_OK) return st;
    if (M == 0 || N == 0) return fail(BG_E_INVALID, "an empty product launches nothing");
    st = resolve_gemm_schedule(d, M, N, K, K, p);
    if (st != BG_OK) return st;
    bg_gemm_schedule s{};
    s.bm = p.bm, s.bn = p.bn, s.bk = p.bk, s.waves_m = p.waves_m, s.waves_n = p.waves_n, s.load_path = p.direct;
    s.group_m = p.group_m, s.stages = p.stages;
    s.last_bm = p.bm2, s.last_bn = p.bn2, s.last_waves_m = p.waves_m2, s.last_waves_n = p.waves_n2;
    s.last_stages = p.stages2;
    *out = s;
    return BG_OK;
}

bg_status bg_gemm_bf16(const bg_gemm_desc* d, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                       const void* B, int64_t ldb, void* C, int64_t ldc, void* ws, size_t ws_bytes,
                       hipStream_t stream)
{
    bg::GemmPlan p{};
    bg_status st = check_gemm_bf16(d, M, N, K, lda, ldb, ldc, p);
    if (st != BG_OK) return st;
    if (M == 0 || N == 0) return BG_OK;
    if (!A || !B || !C) return fail(BG_E_INVALID, "NULL tensor");
    if (!aligned16(A) || !aligned16(B) || !aligned16(C) || lda % 8 || ldb % 8 || ldc % 8)
        return fail(BG_E_ALIGN, "pointers must be 16-byte aligned and leading dimensions multiples of 8");
    if (p.S > 1) {
        const size_t need = (size_t)p.S * (size_t)M * (size_t)N * sizeof(float);
        if (!ws || ws_bytes < need) return fail(BG_E_WORKSPACE, "split-K needs S*M*N*4 bytes of workspace");
        if (!aligned16(ws)) return fail(BG_E_ALIGN, "workspace must be 16-byte aligned");
    }
    st = resolve_gemm_schedule(d, M, N, lda, ldb, p);
    if (st != BG_OK) return st;
    st = check_device();
    if (st != BG_OK) return st;
    hipError_t e = bg::launch_gemm_bf16(p, M, N, K, (const uint16_t*)A, lda, (const uint16_t*)B, ldb, C, ldc,
                                        (float*)ws, stream);
    if (e != hipSuccess) return fail(BG_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
    return BG_OK;
}

bg_status bg_gemm_bf16_noalloc(const bg_gemm_desc* d, int64_t M, int64_t N, int64_t K, const void* A,
                               int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, hipStream_t stream)
{
    size_t need = 0;
    bg_status st = bg_gemm_workspace_bytes(d, M, N, K, &need);
    if (st != BG_OK) return st;
    if (need > kNoallocScratchBytes)
        return fail(BG_E_WORKSPACE, "bg_gemm_bf16_noalloc: the split partials need " + std::to_string(need) +
                                        " bytes; the static scratch holds " + std::to_string(kNoallocScratchBytes));
    void* ws = nullptr;
    if (need > 0 && M > 0 && N > 0) {
        st = check_device();  // the scratch exists only where the gfx950 code object is loaded
        if (st != BG_OK) return st;
        st = scratch_for_current_device(&ws);
        if (st != BG_OK) return st;
    }
    // the same validation, plan and kernels as bg_gemm_bf16, with the
    // scratch as the workspace (every partial is written before it is read,
    // so nothing is cleared)
    return bg_gemm_bf16(d, M, N, K, A, lda, B, ldb, C, ldc, ws, ws ? kNoallocScratchBytes : 0, stream);
}

bg_status bg_gemm_w8a8_pow2(const bg_gemm_desc* d, int64_t M, int64_t N, int64_t K, const int8_t* A,
                            int64_t lda, const int8_t* W, int64_t ldw, const float* a_scale,
                            const float* w_scale, void* Y, int64_t ldy, int32_t* acc_out, int64_t ld_acc,
                            hipStream_t stream)
{
    bg_status st = check_common_order(d);
    if (st != BG_OK) return st;
    if (d->a_type != BG_INT8 || d->b_type != BG_INT8) return fail(BG_E_INVALID, "W8A8 takes int8 operands");
    if (d->acc_type != BG_INT32) return fail(BG_E_INVALID, "W8A8 accumulates in int32");
    if (d->out_type != BG_BF16) return fail(BG_E_INVALID, "W8A8 writes bf16");
    if (d->mfma != BG_MFMA_I32_32X32X32_I8 && d->mfma != BG_MFMA_I32_16X16X64_I8)
        return fail(BG_E_INVALID, "mfma must be an int8 instruction");
    if (d->epilogue != BG_EPI_W8A8_POW2) return fail(BG_E_INVALID, "epilogue must be W8A8_POW2");
    if (d->split_k != 1) return fail(BG_E_UNSUPPORTED, "W8A8 is built with split_k = 1");
    if (M < 0 || N < 0 || K < 1) return fail(BG_E_INVALID, "bad sizes");
    if (K > 131071) return fail(BG_E_UNSUPPORTED, "K > 131071 could leave the exact int32 range");
    if (lda < K || ldw < K || ldy < N || (acc_out && ld_acc < N))
        return fail(BG_E_INVALID, "leading dimension smaller than the row");
    bg::W8A8Plan p{};
    p.mfma = (int)d->mfma;
    const bg_gemm_schedule& s = d->sched;
    p.group_m = s.group_m;
    if (s.bm || s.bn || s.waves_m || s.waves_n) {
        const int path = s.load_path ? s.load_path : 1;
        if (!bg::w8a8_has_tile(p.mfma, s.bm, s.bn, s.waves_m, s.waves_n, path, s.stages))
            return fail(BG_E_UNSUPPORTED, "schedule (bm, bn, waves, load_path, stages) is not compiled in for W8A8");
        // two stages on the pipelined path: 128-byte k tiles, copies addressed
        // by 32-bit offsets (the first compiled entry of a shape, so also
        // stages 0 where the shape has it)
        const bool two = path == 2 && (s.stages == 2 ||
                                       (s.stages == 0 && bg::w8a8_has_tile(p.mfma, s.bm, s.bn, s.waves_m, s.waves_n, 2, 2)));
        if (two && !bg::i8_offsets_fit(s.bm, s.bn, lda, ldw))
            return fail(BG_E_UNSUPPORTED, "a two-stage W8A8 tile addresses its copies by 32-bit offsets: "
                                          "(bm - 1) x lda and (bn - 1) x ldw must stay below 2^32 bytes");
        p.bm = s.bm, p.bn = s.bn, p.waves_m = s.waves_m, p.waves_n = s.waves_n;
        p.path = path, p.stages = two ? 2 : s.stages;
    } else if (p.mfma == BG_MFMA_I32_32X32X32_I8) {
        choose_w8a8_pipe(p, M, N, lda, ldw);
    } else {
        const bool big = M >= 128 && N >= 128 && ((M + 127) / 128) * ((N + 127) / 128) >= 128;
        p.bm = big ? 128 : 64, p.bn = big ? 128 : 64, p.waves_m = 2, p.waves_n = 2;
        p.path = 1, p.stages = 0;
    }
    if (M == 0 || N == 0) return BG_OK;
    if (!A || !W || !a_scale || !w_scale || !Y) return fail(BG_E_INVALID, "NULL tensor");
    if (!aligned16(A) || !aligned16(W) || lda % 16 || ldw % 16 || !aligned16(Y) || ldy % 8 ||
        ((uintptr_t)a_scale & 3u) || ((uintptr_t)w_scale & 3u) || (acc_out && (!aligned16(acc_out) || ld_acc % 4)))
        return fail(BG_E_ALIGN, "pointers must be aligned and leading dimensions multiples of 16 (int8) / 8 / 4");
    if (!tiles_fit(M, N, p.bm, p.bn, 64 * p.waves_m * p.waves_n)) return fail(BG_E_UNSUPPORTED, "M x N too large for one launch");
    st = check_device();
    if (st != BG_OK) return st;
    hipError_t e = bg::launch_w8a8(p, M, N, K, A, lda, W, ldw, a_scale, w_scale, (uint16_t*)Y, ldy, acc_out,
                                   ld_acc, stream);
    if (e != hipSuccess) return fail(BG_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
    return BG_OK;
}

// Validate a reduce descriptor and fill the plan; BG_OK or a refusal.
static bg_status reduce_plan(const bg_reduce_desc* d, int64_t rows, int64_t cols, bg::ReducePlan& p,
                             int64_t& n_blocks)
{
    if (!d) return fail(BG_E_INVALID, "descriptor is NULL");
    if (d->version != 1) return fail(BG_E_INVALID, "descriptor version must be 1");
    if (d->in_type != BG_FP32 && d->in_type != BG_BF16) return fail(BG_E_INVALID, "in_type must be fp32 or bf16");
    if (d->acc_type != BG_FP32 || d->out_type != BG_FP32) return fail(BG_E_INVALID, "accumulation and output are fp32");
    if (d->op < BG_RED_SUM || d->op > BG_RED_SUM_AND_SUMSQ) return fail(BG_E_INVALID, "unknown op");
    if (d->axis != BG_AXIS_ROW && d->axis != BG_AXIS_COL) return fail(BG_E_INVALID, "unknown axis");
    if (d->leaf_order != BG_LEAF_SEQUENTIAL_NO_SEED) return fail(BG_E_INVALID, "unknown leaf_order");
    if (d->sq_fma != BG_SQ_FUSED && d->sq_fma != BG_SQ_UNFUSED) return fail(BG_E_INVALID, "unknown sq_fma");
    if (d->tree != BG_TREE_BALANCED) return fail(BG_E_INVALID, "unknown tree");
    if (d->odd_rule != BG_ODD_CARRY_LAST) return fail(BG_E_INVALID, "unknown odd_rule");
    if (d->leaf_len != 32) return fail(BG_E_UNSUPPORTED, "only leaves of 32 elements are built");
    if (rows < 0 || cols < 0) return fail(BG_E_INVALID, "negative size");
    p.axis = (int)d->axis;
    p.bf16 = d->in_type == BG_BF16;
    p.fused = d->sq_fma == BG_SQ_FUSED;
    if (p.axis == BG_AXIS_ROW) {
        n_blocks = bg::reduce_row_blocks(cols);
        if (n_blocks > 64) return fail(BG_E_UNSUPPORTED, "a row longer than 64 * 8192 elements is not built");
    } else if (d->sched.leaves_per_wg == 256) {
        // one pass, a workgroup per column strip over every row (rows <= 8192)
        if ((rows + 31) / 32 > 256) return fail(BG_E_UNSUPPORTED, "the one-pass column path holds 256 leaves");
        p.col_full = true;
        n_blocks = 1;
    } else {
        // speed only (any aligned run of leaves is an exact subtree): 4
        // leaves per workgroup for bf16 and 8 for fp32 (the fastest at 8192 x
        // 4096 with inputs not in the MALL: 16.2 and 24.0 us), raised until
        // the block roots fit within 64
        int lpw = d->sched.leaves_per_wg;
        if (!lpw) {
            lpw = p.bf16 ? 4 : 8;
            while (lpw < 32 && bg::reduce_col_blocks(rows, lpw) > 64) lpw *= 2;
        }
        p.leaves_per_wg = lpw;
        if (p.leaves_per_wg != 4 && p.leaves_per_wg != 8 && p.leaves_per_wg != 16 && p.leaves_per_wg != 32)
            return fail(BG_E_UNSUPPORTED, "leaves_per_wg must be 4, 8, 16 or 32");
        const int cpw = d->sched.cols_per_wg ? d->sched.cols_per_wg : 256;
        p.cols_per_lane = cpw / 64;
        if (cpw % 64 || (p.cols_per_lane != 4 && (p.cols_per_lane != 8 || !p.bf16)))
            return fail(BG_E_UNSUPPORTED, "cols_per_wg must be 256 (or 512 for bf16 input)");
        n_blocks = bg::reduce_col_blocks(rows, p.leaves_per_wg);
        if (n_blocks > 64)
            return fail(BG_E_UNSUPPORTED, d->sched.leaves_per_wg ? "too many leaf blocks: raise leaves_per_wg"
                                                                 : "a column longer than 64 * 32 leaves (65,536 rows) is not built");
    }
    return BG_OK;
}

bg_status bg_reduce_workspace_bytes(const bg_reduce_desc* d, int64_t rows, int64_t cols, size_t* bytes)
{
    if (!bytes) return fail(BG_E_INVALID, "NULL argument");
    bg::ReducePlan p{};
    int64_t nb = 0;
    bg_status st = reduce_plan(d, rows, cols, p, nb);
    if (st != BG_OK) return st;
    const int64_t n_out = p.axis == BG_AXIS_ROW ? rows : cols;
    *bytes = nb > 1 ? (size_t)n_out * (size_t)nb * 2 * sizeof(float) : 0;
    return BG_OK;
}

bg_status bg_reduce_tree(const bg_reduce_desc* d, int64_t rows, int64_t cols, const void* X, int64_t ldx,
                         float* out_sum, float* out_sumsq, void* ws, size_t ws_bytes, hipStream_t stream)
{
    bg::ReducePlan p{};
    int64_t nb = 0;
    bg_status st = reduce_plan(d, rows, cols, p, nb);
    if (st != BG_OK) return st;
    if (!(d->op & BG_RED_SUM)) out_sum = nullptr;
    if (!(d->op & BG_RED_SUMSQ)) out_sumsq = nullptr;
    if (ldx < cols) return fail(BG_E_INVALID, "leading dimension smaller than the row");
    if (rows == 0 || cols == 0) return BG_OK;
    if (!X) return fail(BG_E_INVALID, "NULL tensor");
    if ((d->op & BG_RED_SUM) && !out_sum) return fail(BG_E_INVALID, "op asks for the sum but out_sum is NULL");
    if ((d->op & BG_RED_SUMSQ) && !out_sumsq) return fail(BG_E_INVALID, "op asks for sumsq but out_sumsq is NULL");
    if (!aligned16(X) || ldx % 8) return fail(BG_E_ALIGN, "X must be 16-byte aligned with ldx a multiple of 8");
    if (((uintptr_t)out_sum & 3u) || ((uintptr_t)out_sumsq & 3u)) return fail(BG_E_ALIGN, "outputs must be 4-byte aligned");
    const int64_t n_out = p.axis == BG_AXIS_ROW ? rows : cols;
    const size_t need = nb > 1 ? (size_t)n_out * (size_t)nb * 2 * sizeof(float) : 0;
    if (need && (!ws || ws_bytes < need)) return fail(BG_E_WORKSPACE, "this shape needs a workspace");
    // row axis: a workgroup per row; column axis: a workgroup per strip of
    // 256 or more columns, or in one pass per strip of 32 (bf16, 512 lanes) or
    // 16 (fp32, 1024 lanes); the upper levels take 256 lanes per 64 outputs
    const bool fits = p.axis == BG_AXIS_ROW ? grid_fits(rows, 256)
                      : p.col_full          ? grid_fits(p.bf16 ? (cols + 31) / 32 : (cols + 15) / 16, p.bf16 ? 512 : 1024)
                                            : grid_fits((cols + 63) / 64, 256);
    if (!fits)
        return fail(BG_E_UNSUPPORTED, "too many rows or columns for one launch");
    st = check_device();
    if (st != BG_OK) return st;
    hipError_t e = bg::launch_reduce(p, rows, cols, X, ldx, out_sum, out_sumsq, (float*)ws, stream);
    if (e != hipSuccess) return fail(BG_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
    return BG_OK;
}

bg_status bg_gemm_bf16_reduce_workspace_bytes(const bg_gemm_desc* d, const bg_reduce_desc* rd, int64_t M,
                                              int64_t N, int64_t K, size_t* bytes)
{
    (void)K;
    if (!d || !bytes) return fail(BG_E_INVALID, "NULL argument");
    bg_status st = check_fused_reduce(rd);
    if (st != BG_OK) return st;
    if (M < 0 || N < 0) return fail(BG_E_INVALID, "negative size");
    int64_t n_leaf, n_out;
    fused_reduce_shape(rd, M, N, n_leaf, n_out, *bytes);
    return BG_OK;
}

bg_status bg_gemm_bf16_reduce(const bg_gemm_desc* d, const bg_reduce_desc* rd, int64_t M, int64_t N, int64_t K,
                              const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                              float* out_sum, float* out_sumsq, void* ws, size_t ws_bytes, hipStream_t stream)
{
    bg_status st = check_common_order(d);
    if (st != BG_OK) return st;
    if (d->a_type != BG_BF16 || d->b_type != BG_BF16) return fail(BG_E_INVALID, "bf16 operands");
    if (d->acc_type != BG_FP32) return fail(BG_E_INVALID, "bf16 GEMM accumulates in fp32");
    if (d->out_type != BG_FP32 && d->out_type != BG_BF16) return fail(BG_E_INVALID, "out_type must be fp32 or bf16");
    if (d->mfma != BG_MFMA_F32_32X32X16_BF16)
        return fail(BG_E_UNSUPPORTED, "the fused reductions are built for the 32x32x16 instruction");
    if (d->partial_type != BG_FP32 || d->merge_type != BG_FP32)
        return fail(BG_E_UNSUPPORTED, "only fp32 partials merged in fp32 are built");
    if (d->combine != BG_COMBINE_BALANCED) return fail(BG_E_UNSUPPORTED, "only the balanced combine is built");
    if (d->epilogue != BG_EPI_NONE) return fail(BG_E_INVALID, "bg_gemm_bf16_reduce has no other epilogue");
    if (d->split_k != 1) return fail(BG_E_UNSUPPORTED, "the fused reductions take split_k 1");
    st = check_fused_reduce(rd);
    if (st != BG_OK) return st;
    if (M < 0 || N < 0 || K < 1) return fail(BG_E_INVALID, "bad sizes");
    if (lda < K || ldb < K || ldc < N) return fail(BG_E_INVALID, "leading dimension smaller than the row");
    // the split is [0, K): its end is a cut point, which the kernels take in
    // whole 16-byte chunks (as bg_gemm_bf16 requires of every cut point)
    if (K % 8) return fail(BG_E_UNSUPPORTED, "K must be a multiple of 8 (the cut point at K)");
    if (!(rd->op & BG_RED_SUM)) out_sum = nullptr;
    if (!(rd->op & BG_RED_SUMSQ)) out_sumsq = nullptr;
    int64_t n_leaf, n_out;
    size_t need;
    fused_reduce_shape(rd, M, N, n_leaf, n_out, need);
    if (n_leaf > 1024) return fail(BG_E_UNSUPPORTED, "the reduced axis holds at most 1024 leaves (32768 elements)");
    if (M == 0 || N == 0) return BG_OK;
    if (!A || !B || !C) return fail(BG_E_INVALID, "NULL tensor");
    if ((rd->op & BG_RED_SUM) && !out_sum) return fail(BG_E_INVALID, "op asks for the sum but out_sum is NULL");
    if ((rd->op & BG_RED_SUMSQ) && !out_sumsq) return fail(BG_E_INVALID, "op asks for sumsq but out_sumsq is NULL");
    if (!aligned16(A) || !aligned16(B) || !aligned16(C) || lda % 8 || ldb % 8 || ldc % 8)
        return fail(BG_E_ALIGN, "pointers must be 16-byte aligned and leading dimensions multiples of 8");
    if (((uintptr_t)out_sum & 3u) || ((uintptr_t)out_sumsq & 3u)) return fail(BG_E_ALIGN, "outputs must be 4-byte aligned");
    if (!ws || ws_bytes < need) return fail(BG_E_WORKSPACE, "the fused reductions need a workspace");
    if ((uintptr_t)ws & 3u) return fail(BG_E_ALIGN, "workspace must be 4-byte aligned");

    bg::GemmPlan p{};
    p.S = 1;
    p.cuts.c[0] = 0;
    p.cuts.c[1] = K;
    p.mfma = (int)d->mfma;
    p.out_bf16 = d->out_type == BG_BF16;
    const bg_gemm_schedule& s = d->sched;
    p.group_m = s.group_m;
    if (s.bm || s.bn || s.bk || s.waves_m || s.waves_n) {
        const int bk = s.bk ? s.bk : 32;
        if ((s.load_path && s.load_path != 2) ||
            !bg::gemm_bf16_red_has_tile(s.bm, s.bn, bk, s.waves_m, s.waves_n, s.stages))
            return fail(BG_E_UNSUPPORTED, "schedule is not built with the fused reductions");
        if (bk == 64 && !bg::pipe_offsets_fit(s.bm, s.bn, lda, ldb))
            return fail(BG_E_UNSUPPORTED, "a 64-deep pipelined tile addresses its copies by 32-bit offsets: "
                                          "(bm - 1) x lda and (bn - 1) x ldb must stay below 2^31 elements");
        p.bm = s.bm, p.bn = s.bn, p.bk = bk, p.waves_m = s.waves_m, p.waves_n = s.waves_n, p.direct = 2;
        p.stages = s.stages;
    } else {  // speed only: the tiles built with the reductions
        auto set = [&](int bm, int bn, int bk, int wm, int wn, int ns) {
            p.bm = bm, p.bn = bn, p.bk = bk, p.waves_m = wm, p.waves_n = wn, p.direct = 2, p.stages = ns;
        };
        const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
        if (big >= 384) {
            if (bg::pipe_offsets_fit(320, 256, lda, ldb)) set(320, 256, 64, 2, 4, 2);
            else set(320, 256, 32, 2, 4, 4);
        } else if (M > 64 && ((M + 255) / 256) * ((N + 127) / 128) >= 150) {
            set(256, 128, 32, 2, 2, 4);
        } else {
            set(64, 64, 32, 2, 2, 8);
        }
    }
    if (!tiles_fit(M, N, p.bm, p.bn, 64 * p.waves_m * p.waves_n) || !grid_fits((n_out + 63) / 64, 1024))
        return fail(BG_E_UNSUPPORTED, "M x N too large for one launch");
    float* ws_sum = (float*)ws;
    float* ws_sq = (float*)ws + ((rd->op & BG_RED_SUM) ? n_leaf * n_out : 0);
    p.red = rd->axis == BG_AXIS_COL ? 1 : 2;
    p.red_args.ws_sum = out_sum ? ws_sum : nullptr;
    p.red_args.ws_sq = out_sumsq ? ws_sq : nullptr;
    p.red_args.n_out = n_out;
    p.red_args.fused = rd->sq_fma == BG_SQ_FUSED;
    st = check_device();
    if (st != BG_OK) return st;
    hipError_t e = bg::launch_gemm_bf16_reduce(p, M, N, (const uint16_t*)A, lda, (const uint16_t*)B, ldb, C, ldc,
                                               stream);
    if (e == hipSuccess)
        e = bg::launch_leaf_tree(p.red_args.ws_sum, p.red_args.ws_sq, n_out, (int)n_leaf, out_sum, out_sumsq, stream);
    if (e != hipSuccess) return fail(BG_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
    return BG_OK;
}

static size_t align16z(size_t x) { return (x + 15) & ~(size_t)15; }

// slicing: a workgroup per row of A and of B; the stacked product 4M x 4N
bool ozaki_fits(int64_t M, int64_t N)
{
    return grid_fits(M, 256) && grid_fits(N, 256) && grid_fits((M * N + 255) / 256, 256);
}

bg_status bg_gemm_ozaki_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes)
{
    if (!bytes) return fail(BG_E_INVALID, "NULL argument");
    if (M < 0 || N < 0 || K < 0) return fail(BG_E_INVALID, "negative size");
    if (!ozaki_fits(M, N)) return fail(BG_E_UNSUPPORTED, "M, N below 2^24 and M x N below 2^32 for one launch");
    const size_t Kp = (size_t)((K + 15) / 16 * 16);
    *bytes = align16z(4 * (size_t)M * Kp) + align16z(4 * (size_t)N * Kp) + align16z(4 * (size_t)M) +
             align16z(4 * (size_t)N);
    return BG_OK;
}

bg_status bg_gemm_ozaki(int64_t M, int64_t N, int64_t K, uint32_t in_type, const void* A, int64_t lda,
                        const void* B, int64_t ldb, uint32_t out_type, void* C, int64_t ldc, void* ws,
                        size_t ws_bytes, hipStream_t stream)
{
    if (in_type != BG_FP32 && in_type != BG_BF16) return fail(BG_E_INVALID, "in_type must be fp32 or bf16");
    if (out_type != BG_FP32 && out_type != BG_BF16) return fail(BG_E_INVALID, "out_type must be fp32 or bf16");
    if (M < 0 || N < 0 || K < 0) return fail(BG_E_INVALID, "negative size");
    if (!ozaki_fits(M, N)) return fail(BG_E_UNSUPPORTED, "M, N below 2^24 and M x N below 2^32 for one launch");
    const int64_t Kp = (K + 15) / 16 * 16;
    if (Kp > 133144) return fail(BG_E_UNSUPPORTED, "K rounded up to 16 above 133,144 could leave the int32 range");
    if (lda < K || ldb < K || ldc < N) return fail(BG_E_INVALID, "leading dimension smaller than the row");
    if (M == 0 || N == 0) return BG_OK;
    if (!A || !B || !C) return fail(BG_E_INVALID, "NULL tensor");
    const uintptr_t ea = in_type == BG_BF16 ? 1u : 3u, ec = out_type == BG_BF16 ? 1u : 3u;
    if (((uintptr_t)A & ea) || ((uintptr_t)B & ea) || ((uintptr_t)C & ec))
        return fail(BG_E_ALIGN, "A, B and C must be aligned to their element size");
    size_t need = 0;
    (void)bg_gemm_ozaki_workspace_bytes(M, N, K, &need);
    if (!ws || ws_bytes < need) return fail(BG_E_WORKSPACE, "the Ozaki GEMM needs a workspace");
    if (!aligned16(ws)) return fail(BG_E_ALIGN, "workspace must be 16-byte aligned");
    bg::OzakiWs w{};
    w.Kp = Kp;
    char* base = (char*)ws;
    w.qa = (int8_t*)base;
    base += align16z(4 * (size_t)M * (size_t)Kp);
    w.qb = (int8_t*)base;
    base += align16z(4 * (size_t)N * (size_t)Kp);
    w.ea = (int*)base;
    base += align16z(4 * (size_t)M);
    w.eb = (int*)base;
    // speed only: the pipelined int8 tiles (every shape gives the same integers)
    bg::W8A8Plan p{};
    p.mfma = BG_MFMA_I32_32X32X32_I8;
    choose_w8a8_pipe(p, 4 * M, 4 * N, Kp, Kp);
    if (!bg::w8a8_ozaki_has_tile(p) || !tiles_fit(4 * M, 4 * N, p.bm, p.bn, 64 * p.waves_m * p.waves_n))
        return fail(BG_E_UNSUPPORTED, "M x N too large for one launch");
    bg_status st = check_device();
    if (st != BG_OK) return st;
    hipError_t e = bg::launch_ozaki(p, M, N, K, in_type == BG_BF16, A, lda, B, ldb, out_type == BG_BF16, C, ldc, w,
                                    stream);
    if (e != hipSuccess) return fail(BG_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
    return BG_OK;
}

bg_status bg_quantize_act_int8(int64_t M, int64_t K, const float* X, int64_t ldx, int8_t* Q, int64_t ldq,
                               float* a_scale, hipStream_t stream)
{
    if (M < 0 || K < 0) return fail(BG_E_INVALID, "negative size");
    if (!grid_fits(M, 256)) return fail(BG_E_UNSUPPORTED, "at most 2^24 - 1 rows (a workgroup per row)");
    if (ldx < K || ldq < K) return fail(BG_E_INVALID, "leading dimension smaller than the row");
    if (M == 0) return BG_OK;
    if (!a_scale || (K > 0 && (!X || !Q))) return fail(BG_E_INVALID, "NULL tensor");
    if (((uintptr_t)X & 3u) || ((uintptr_t)a_scale & 3u)) return fail(BG_E_ALIGN, "X and a_scale must be 4-byte aligned");
    bg_status st = check_device();
    if (st != BG_OK) return st;
    const bool vec = aligned16(X) && ldx % 4 == 0 && K % 4 == 0 && ((uintptr_t)Q & 3u) == 0 && ldq % 4 == 0;
    hipError_t e = bg::launch_quantize_rows(M, K, X, ldx, Q, ldq, a_scale, vec, stream);
    if (e != hipSuccess) return fail(BG_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
    return BG_OK;
}

bg_status bg_requantize_weights_pow2(int64_t N, int64_t K, const int8_t* W, int64_t ldw, const float* w_scale,
                                     uint32_t mode, int8_t* W2, int64_t ldw2, float* w_scale2,
                                     hipStream_t stream)
{
    if (N < 0 || K < 0) return fail(BG_E_INVALID, "negative size");
    if (!grid_fits((N + 1) / 2, 256)) return fail(BG_E_UNSUPPORTED, "at most 2^25 - 2 rows (a workgroup per two rows)");
    if (mode != BG_POW2_NEAREST && mode != BG_POW2_CEIL) return fail(BG_E_INVALID, "unknown mode");
    if (ldw < K || ldw2 < K) return fail(BG_E_INVALID, "leading dimension smaller than the row");
    if (N == 0) return BG_OK;
    if (!w_scale || !w_scale2 || (K > 0 && (!W || !W2))) return fail(BG_E_INVALID, "NULL tensor");
    if (((uintptr_t)w_scale & 3u) || ((uintptr_t)w_scale2 & 3u)) return fail(BG_E_ALIGN, "scales must be 4-byte aligned");
    const uintptr_t w0 = (uintptr_t)W, w1 = w0 + (uintptr_t)((N - 1) * ldw + K);
    const uintptr_t o0 = (uintptr_t)W2, o1 = o0 + (uintptr_t)((N - 1) * ldw2 + K);
    if (K > 0 && w0 < o1 && o0 < w1) return fail(BG_E_INVALID, "W2 may not overlap W");
    bg_status st = check_device();
    if (st != BG_OK) return st;
    const bool vec = aligned16(W) && aligned16(W2) && ldw % 16 == 0 && ldw2 % 16 == 0 && K % 16 == 0;
    hipError_t e = bg::launch_requantize_pow2(N, K, W, ldw, w_scale, (int)mode, W2, ldw2, w_scale2, vec, stream);
    if (e != hipSuccess) return fail(BG_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
    return BG_OK;
}

bg_status bg_bench_gemm_bf16_free(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                                  int64_t ldb, float* C, int64_t ldc, int32_t split_k, hipStream_t stream)
{
    if (M < 0 || N < 0 || K < 1) return fail(BG_E_INVALID, "bad sizes");
    if (lda < K || ldb < K || ldc < N) return fail(BG_E_INVALID, "leading dimension smaller than the row");
    if (split_k > BG_MAX_SPLIT) return fail(BG_E_INVALID, "split_k must be at most 64");
    if (M == 0 || N == 0) return BG_OK;
    if (!A || !B || !C) return fail(BG_E_INVALID, "NULL tensor");
    if (!aligned16(A) || !aligned16(B) || !aligned16(C) || lda % 8 || ldb % 8 || ldc % 8)
        return fail(BG_E_ALIGN, "pointers must be 16-byte aligned and leading dimensions multiples of 8");
    bg_status st = check_device();
    if (st != BG_OK) return st;
    bg::GemmPlan p{};
    p.mfma = BG_MFMA_F32_32X32X16_BF16;
    p.out_bf16 = false;
    p.S = 1;
    p.cuts.c[0] = 0;
    p.cuts.c[1] = K;
    choose_gemm_tile(p, M, N, lda, ldb);
    int S = split_k;
    if (S <= 0) {  // at least one workgroup per CU, each split at least 256 deep
        int dev = 0, n_cu = 256;
        if (hipGetDevice(&dev) == hipSuccess)
            (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        const int64_t tiles = ((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
        S = 1;
        while (S < BG_MAX_SPLIT && tiles * S < n_cu && K / (2 * S) >= 256) S *= 2;
    }
    const int64_t span = (K / (64 * (int64_t)S)) * 64;
    if (S > 1 && span == 0) return fail(BG_E_INVALID, "K too small for that many splits");
    p.S = S;
    for (int s = 0; s < S; s++) p.cuts.c[s] = s * span;
    p.cuts.c[S] = K;
    p.atomic = S > 1;
    if (S > 1) choose_gemm_tile(p, M, N, lda, ldb);  // the tile (or pair of tiles) for the split grid
    if (!tiles_fit(M, N, p.bm, p.bn, 64 * p.waves_m * p.waves_n))
        return fail(BG_E_UNSUPPORTED, "M x N too large for one launch");
    p.atomic = S > 1;
    hipError_t e = hipSuccess;
    if (p.atomic) e = bg::launch_zero_rows(C, M, N, ldc, stream);
    if (e == hipSuccess)
        e = bg::launch_gemm_bf16(p, M, N, K, (const uint16_t*)A, lda, (const uint16_t*)B, ldb, C, ldc, nullptr,
                                 stream);
    if (e != hipSuccess) return fail(BG_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
    return BG_OK;
}

bg_status bg_bench_gemm_bf16_two_chains(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                        const void* B, int64_t ldb, float* C, int64_t ldc, hipStream_t stream)
{
    if (M < 0 || N < 0 || K < 1) return fail(BG_E_INVALID, "bad sizes");
    if (lda < K || ldb < K || ldc < N) return fail(BG_E_INVALID, "leading dimension smaller than the row");
    if (K % 8) return fail(BG_E_UNSUPPORTED, "K must be a multiple of 8");
    if (M == 0 || N == 0) return BG_OK;
    if (!A || !B || !C) return fail(BG_E_INVALID, "NULL tensor");
    if (!aligned16(A) || !aligned16(B) || !aligned16(C) || lda % 8 || ldb % 8 || ldc % 8)
        return fail(BG_E_ALIGN, "pointers must be 16-byte aligned and leading dimensions multiples of 8");
    if (!bg::pipe_offsets_fit(128, 128, lda, ldb))
        return fail(BG_E_UNSUPPORTED, "leading dimensions too large for the tile's 32-bit copy offsets");
    if (!tiles_fit(M, N, 128, 128, 256)) return fail(BG_E_UNSUPPORTED, "M x N too large for one launch");
    bg_status st = check_device();
    if (st != BG_OK) return st;
    hipError_t e = bg::launch_gemm_bf16_two_chains(M, N, K, (const uint16_t*)A, lda, (const uint16_t*)B, ldb, C, ldc,
                                                  stream);
    if (e != hipSuccess) return fail(BG_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
    return BG_OK;
}

bg_status bg_bench_gemm_w8a8_free(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda, const int8_t* W,
                                  int64_t ldw, const float* a_scale, const float* w_scale, void* Y, int64_t ldy,
                                  hipStream_t stream)
{
    if (M < 0 || N < 0 || K < 1 || K > 131071) return fail(BG_E_INVALID, "bad sizes");
    if (lda < K || ldw < K || ldy < N) return fail(BG_E_INVALID, "leading dimension smaller than the row");
    if (M == 0 || N == 0) return BG_OK;
    if (!A || !W || !a_scale || !w_scale || !Y) return fail(BG_E_INVALID, "NULL tensor");
    if (!aligned16(A) || !aligned16(W) || lda % 16 || ldw % 16 || !aligned16(Y) || ldy % 8 ||
        ((uintptr_t)a_scale & 3u) || ((uintptr_t)w_scale & 3u))
        return fail(BG_E_ALIGN, "pointers must be aligned and leading dimensions multiples of 16 (int8) / 8");
    bg::W8A8Plan p{};
    p.mfma = BG_MFMA_I32_32X32X32_I8;
    choose_w8a8_pipe(p, M, N, lda, ldw);  // the same tile and main loop as bg_gemm_w8a8_pow2
    p.free_epilogue = true;
    if (!tiles_fit(M, N, p.bm, p.bn, 64 * p.waves_m * p.waves_n)) return fail(BG_E_UNSUPPORTED, "M x N too large for one launch");
    bg_status st = check_device();
    if (st != BG_OK) return st;
    hipError_t e = bg::launch_w8a8(p, M, N, K, A, lda, W, ldw, a_scale, w_scale, (uint16_t*)Y, ldy, nullptr, 0, stream);
    if (e != hipSuccess) return fail(BG_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
    return BG_OK;
}

bg_status bg_bench_reduce_free(uint32_t axis, uint32_t in_type, int64_t rows, int64_t cols, const void* X,
                               int64_t ldx, float* out_sum, float* out_sumsq, hipStream_t stream)
{
    if (axis != BG_AXIS_ROW && axis != BG_AXIS_COL) return fail(BG_E_INVALID, "unknown axis");
    if (in_type != BG_FP32 && in_type != BG_BF16) return fail(BG_E_INVALID, "in_type must be fp32 or bf16");
    if (rows < 0 || cols < 0 || ldx < cols) return fail(BG_E_INVALID, "bad sizes");
    if (rows == 0 || cols == 0) return BG_OK;
    if (!X || !aligned16(X) || ldx % 8) return fail(BG_E_ALIGN, "X must be 16-byte aligned with ldx a multiple of 8");
    if (!grid_fits(axis == BG_AXIS_ROW ? rows : (cols + 511) / 512, 256))
        return fail(BG_E_UNSUPPORTED, "too many rows or columns for one launch");
    bg_status st = check_device();
    if (st != BG_OK) return st;
    int dev = 0, n_cu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    hipError_t e = bg::launch_reduce_free((int)axis, in_type == BG_BF16, rows, cols, X, ldx, out_sum, out_sumsq,
                                          n_cu, stream);
    if (e != hipSuccess) return fail(BG_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
    return BG_OK;
}

bg_status bg_probe_mfma(uint32_t mfma, int64_t n_cases, const void* A, const void* B, const void* C, void* D,
                        hipStream_t stream)
{
    if (instruction_k(mfma) == 0) return fail(BG_E_INVALID, "unknown mfma");
    if (n_cases < 0) return fail(BG_E_INVALID, "n_cases out of range");
    if (!grid_fits(n_cases, 64)) return fail(BG_E_UNSUPPORTED, "at most 2^26 - 1 cases per launch");
    if (n_cases == 0) return BG_OK;
    if (!A || !B || !C || !D) return fail(BG_E_INVALID, "NULL tensor");
    if (!aligned16(A) || !aligned16(B) || !aligned16(C) || !aligned16(D))
        return fail(BG_E_ALIGN, "probe tiles must be 16-byte aligned");
    bg_status st = check_device();
    if (st != BG_OK) return st;
    hipError_t e = bg::launch_probe((int)mfma, n_cases, A, B, C, D, stream);
    if (e != hipSuccess) return fail(BG_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
    return BG_OK;
}

}  // extern "C"
