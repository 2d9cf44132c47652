/* Runs every oracle function on small seeded inputs under AddressSanitizer
 * and UndefinedBehaviorSanitizer (the test builds it with
 * -fsanitize=address,undefined): every array is allocated at exactly the
 * size the oracle documents, so a read or write one element past any of
 * them stops the program.  Shapes cover T = 0, ragged rows, k = 1, k = E,
 * R = 1, E = R and the widest histogram; bad ids must be refused with
 * OR_E_BAD_INDEX.  Prints "ok" and returns 0 when nothing was reported. */
#include "../../oracle/oracle.c"

#include <stdio.h>
#include <string.h>

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void)
{
    /* xorshift64* */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}

/* exactly n elements (n == 0 still gets a distinct, unusable allocation) */
static void* alloc(size_t n, size_t elem) { return malloc(n ? n * elem : 1); }

static void fill_bf16(uint16_t* a, size_t n)
{
    for (size_t i = 0; i < n; ++i) {
        const uint32_t r = next_u32();
        const uint16_t exp = (uint16_t)(100 + r % 50); /* finite, no NaN or Inf */
        a[i] = (uint16_t)(((r >> 8) & 0x8000u) | (exp << 7) | ((r >> 16) & 0x7f));
    }
}

static int run_case(int T, int H, int E, int k, int R, int bad)
{
    oracle_dims d = {T, H, E, k, R};
    if (oracle_check_dims(&d) != OR_OK) return 1;
    const int Epr = E / R, KR = imin(k, R), D = imin(k, Epr);
    const size_t Tk = (size_t)T * k, TKR = (size_t)T * KR;

    int32_t* idx = alloc(Tk, sizeof(int32_t));
    float* w = alloc(Tk, sizeof(float));
    int32_t* perm = alloc((size_t)E, sizeof(int32_t));
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) perm[e] = e;
        for (int j = 0; j < k; ++j) { /* partial Fisher-Yates: k distinct ids */
            const int s = j + (int)(next_u32() % (uint32_t)(E - j));
            const int tmp = perm[j];
            perm[j] = perm[s];
            perm[s] = tmp;
            idx[(size_t)t * k + j] = perm[j];
            w[(size_t)t * k + j] = (float)(next_u32() % 1000) / 997.0f - 0.5f;
        }
    }
    if (bad == 1 && T > 0) idx[(size_t)(T - 1) * k] = E;                       /* out of range */
    if (bad == 2 && T > 0 && k > 1) idx[1] = idx[0];                            /* repeated id */

    oracle_plan_out o;
    o.expert_count = alloc((size_t)E, sizeof(int32_t));
    o.expert_offset = alloc((size_t)E + 1, sizeof(int32_t));
    o.rank_count = alloc((size_t)R, sizeof(int32_t));
    o.rank_offset = alloc((size_t)R + 1, sizeof(int32_t));
    o.send_token = alloc(TKR, sizeof(int32_t));
    o.tok_rank_row = alloc(TKR, sizeof(int32_t));
    o.fan_src = alloc(Tk, sizeof(int32_t));
    o.fan_dst = alloc(TKR * D, sizeof(int32_t));
    o.comb_row = alloc(Tk, sizeof(int32_t));
    o.rank_segs = alloc((size_t)R * 4, sizeof(int32_t));
    o.expert_segs = alloc((size_t)E * 4, sizeof(int32_t));
    o.n_rank_rows = alloc(1, sizeof(int32_t));

    int failed = 0;
    const int rc = oracle_plan(&d, idx, &o);
    if (bad && T > 0 && (bad == 1 || k > 1)) {
        failed = rc != OR_E_BAD_INDEX;
    } else if (rc != OR_OK) {
        failed = 1;
    } else {
        const int32_t N = o.n_rank_rows[0];
        uint16_t* x = alloc((size_t)T * H, sizeof(uint16_t));
        uint16_t* xr = alloc((size_t)N * H, sizeof(uint16_t));
        uint16_t* xe = alloc(Tk * H, sizeof(uint16_t));
        uint16_t* out = alloc((size_t)T * H, sizeof(uint16_t));
        uint16_t* g = alloc((size_t)T * H, sizeof(uint16_t));
        uint16_t* gye = alloc(Tk * H, sizeof(uint16_t));
        uint16_t* gxr = alloc((size_t)N * H, sizeof(uint16_t));
        uint16_t* gx = alloc((size_t)T * H, sizeof(uint16_t));
        uint16_t* part = alloc((size_t)N * H, sizeof(uint16_t));
        float* part32 = alloc((size_t)N * H, sizeof(float));
        double* gw = alloc(Tk, sizeof(double));
        fill_bf16(x, (size_t)T * H);
        fill_bf16(g, (size_t)T * H);
        failed |= oracle_dispatch(&d, o.send_token, o.fan_src, N, x, xr, xe) != OR_OK;
        failed |= oracle_combine(&d, o.comb_row, xe, w, out) != OR_OK;
        failed |= oracle_dispatch_backward(&d, o.fan_dst, o.tok_rank_row, N, xe, gxr, gx) != OR_OK;
        failed |= oracle_combine_backward(&d, o.comb_row, g, xe, w, gye, gw) != OR_OK;
        failed |= oracle_combine_rank_partial(&d, o.fan_dst, o.tok_rank_row, o.comb_row, N, xe, w, part, out) !=
                  OR_OK;
        failed |= oracle_combine_rank_partial_f32(&d, o.fan_dst, o.tok_rank_row, o.comb_row, N, xe, w, part32,
                                                  out) != OR_OK;
        free(x); free(xr); free(xe); free(out); free(g); free(gye); free(gxr); free(gx); free(part);
        free(part32); free(gw);
    }
    free(o.expert_count); free(o.expert_offset); free(o.rank_count); free(o.rank_offset);
    free(o.send_token); free(o.tok_rank_row); free(o.fan_src); free(o.fan_dst); free(o.comb_row);
    free(o.rank_segs); free(o.expert_segs); free(o.n_rank_rows);
    free(idx); free(w); free(perm);
    if (failed) printf("case T=%d H=%d E=%d k=%d R=%d bad=%d failed\n", T, H, E, k, R, bad);
    return failed;
}

int main(void)
{
    static const int shapes[][5] = {
        /* T, H, E, k, R */
        {0, 8, 8, 2, 4},     {1, 8, 8, 2, 4},      {63, 136, 8, 3, 4},   {65, 24, 16, 4, 4},
        {130, 16, 32, 8, 8}, {77, 8, 12, 12, 3},   {50, 40, 6, 1, 6},    {40, 8, 16, 16, 1},
        {33, 16, 960, 8, 64}, {20, 8, 128, 64, 8}, {17, 8, 1, 1, 1},     {200, 64, 64, 6, 16},
    };
    int failed = 0;
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
        for (int bad = 0; bad < 3; ++bad)
            failed |= run_case(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], shapes[i][4], bad);
    if (failed) return 1;
    printf("ok\n");
    return 0;
}
