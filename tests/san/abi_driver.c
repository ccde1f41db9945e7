/* Drives every entry point of include/gdn.h through its rejection paths and
 * its accepted paths (host validation only: the launchers are stand-ins).
 * Built with the address and undefined-behaviour sanitizers; any report
 * aborts the run.  Prints one line per check and exits non-zero on a wrong
 * status code. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdn.h"

extern int g_launches;
static int failures = 0;

static void expect(const char *what, int got, int want) {
    const char *msg = gdn_last_error();
    if (got != want) {
        printf("FAIL %s: status %d, want %d (%s)\n", what, got, want, msg);
        ++failures;
    } else {
        printf("ok   %s: %d (%s)\n", what, got, msg && msg[0] ? msg : "-");
    }
}

static gdn_shape shape(int B, int T, int H, int dk, int dv, int chunk, int n_seqs, int io,
                       int o, int pro) {
    gdn_shape s;
    memset(&s, 0, sizeof s);
    s.B = B; s.T = T; s.H = H; s.d_k = dk; s.d_v = dv; s.chunk = chunk; s.n_seqs = n_seqs;
    s.io_dtype = io; s.o_dtype = o; s.prologue = pro;
    return s;
}

int main(void) {
    /* aligned fake device addresses (never dereferenced on the host) */
    void *q = (void *)0x10000, *k = (void *)0x20000, *v = (void *)0x30000;
    float *la = (float *)0x40000, *be = (float *)0x50000, *S0 = (float *)0x60000;
    void *o = (void *)0x70000;
    float *ST = (float *)0x80000;
    const int32_t *cu = (const int32_t *)0x90000;
    void *ws = (void *)0xa0000, *mis = (void *)0x10004;
    void *dq = (void *)0xb0000, *dk = (void *)0xc0000, *dv = (void *)0xd0000;
    float *dla = (float *)0xe0000, *dbe = (float *)0xf0000, *dS0 = (float *)0x100000;
    size_t bytes = 0;
    gdn_shape s = shape(2, 100, 4, 128, 128, 64, 0, GDN_BF16, GDN_F32, 0);

    printf("version %s\n", gdn_version());
    /* forward */
    expect("fwd ws null shape", gdn_chunk_fwd_workspace_size(NULL, &bytes), GDN_ERR_INVALID_ARG);
    expect("fwd ws null out", gdn_chunk_fwd_workspace_size(&s, NULL), GDN_ERR_INVALID_ARG);
    expect("fwd ws", gdn_chunk_fwd_workspace_size(&s, &bytes), GDN_OK);
    gdn_shape bad = s; bad.B = 0;
    expect("fwd bad B", gdn_chunk_fwd(&bad, q, k, v, la, be, S0, NULL, o, ST, NULL, 0, NULL),
           GDN_ERR_INVALID_ARG);
    bad = s; bad.d_v = 96;
    expect("fwd unsupported", gdn_chunk_fwd(&bad, q, k, v, la, be, S0, NULL, o, ST, NULL, 0, NULL),
           GDN_ERR_UNSUPPORTED);
    bad = s; bad.io_dtype = 7;
    expect("fwd bad dtype", gdn_chunk_fwd(&bad, q, k, v, la, be, S0, NULL, o, ST, NULL, 0, NULL),
           GDN_ERR_INVALID_ARG);
    bad = s; bad.prologue = 8;
    expect("fwd bad prologue", gdn_chunk_fwd(&bad, q, k, v, la, be, S0, NULL, o, ST, NULL, 0, NULL),
           GDN_ERR_INVALID_ARG);
    bad = s; bad.n_seqs = 3;
    expect("fwd varlen B>1", gdn_chunk_fwd(&bad, q, k, v, la, be, S0, cu, o, ST, NULL, 0, NULL),
           GDN_ERR_INVALID_ARG);
    expect("fwd misaligned", gdn_chunk_fwd(&s, mis, k, v, la, be, S0, NULL, o, ST, NULL, 0, NULL),
           GDN_ERR_ALIGNMENT);
    expect("fwd alias", gdn_chunk_fwd(&s, q, k, v, la, be, S0, NULL, q, ST, NULL, 0, NULL),
           GDN_ERR_INVALID_ARG);
    expect("fwd missing q", gdn_chunk_fwd(&s, NULL, k, v, la, be, S0, NULL, o, ST, NULL, 0, NULL),
           GDN_ERR_INVALID_ARG);
    expect("fwd cu without n_seqs", gdn_chunk_fwd(&s, q, k, v, la, be, S0, cu, o, ST, NULL, 0, NULL),
           GDN_ERR_INVALID_ARG);
    int before = g_launches;
    expect("fwd ok", gdn_chunk_fwd(&s, q, k, v, la, be, S0, NULL, o, ST, NULL, 0, NULL), GDN_OK);
    gdn_shape f32 = shape(1, 64, 1, 16, 16, 16, 0, GDN_F32, GDN_F32, 3);
    expect("fwd f32 ok", gdn_chunk_fwd(&f32, q, k, v, la, be, NULL, NULL, o, ST, NULL, 0, NULL),
           GDN_OK);
    gdn_shape vl = shape(1, 300, 2, 64, 64, 64, 5, GDN_BF16, GDN_BF16, 0);
    expect("fwd varlen ok", gdn_chunk_fwd(&vl, q, k, v, la, be, S0, cu, o, ST, NULL, 0, NULL),
           GDN_OK);
    gdn_shape empty = shape(2, 0, 4, 128, 128, 64, 0, GDN_BF16, GDN_F32, 0);
    expect("fwd empty", gdn_chunk_fwd(&empty, NULL, NULL, NULL, NULL, NULL, S0, NULL, NULL, ST,
                                      NULL, 0, NULL), GDN_OK);
    if (g_launches <= before) { printf("FAIL fwd: no launch reached\n"); ++failures; }

    /* backward */
    expect("bwd ws", gdn_chunk_bwd_workspace_size(&s, &bytes), GDN_OK);
    expect("bwd small ws", gdn_chunk_bwd(&s, q, k, v, la, be, S0, NULL, o, NULL, dq, dk, dv, dla,
                                         dbe, dS0, ws, bytes - 1, NULL), GDN_ERR_WORKSPACE);
    expect("bwd alias", gdn_chunk_bwd(&s, q, k, v, la, be, S0, NULL, o, NULL, q, dk, dv, dla,
                                      dbe, dS0, ws, bytes, NULL), GDN_ERR_INVALID_ARG);
    expect("bwd prologue", gdn_chunk_bwd_workspace_size(&f32, &bytes), GDN_ERR_UNSUPPORTED);
    expect("bwd ws", gdn_chunk_bwd_workspace_size(&s, &bytes), GDN_OK);
    expect("bwd ok", gdn_chunk_bwd(&s, q, k, v, la, be, S0, NULL, o, NULL, dq, dk, dv, dla, dbe,
                                   dS0, ws, bytes, NULL), GDN_OK);

    /* channel-wise decay, with and without a caller workspace */
    expect("kda ws", gdn_kda_fwd_workspace_size(&s, &bytes), GDN_OK);
    expect("kda null ws", gdn_kda_fwd(&s, q, k, v, la, be, S0, NULL, o, ST, NULL, bytes, NULL),
           GDN_ERR_WORKSPACE);
    expect("kda ok", gdn_kda_fwd(&s, q, k, v, la, be, S0, NULL, o, ST, ws, bytes, NULL), GDN_OK);
    expect("kda noalloc ok", gdn_kda_fwd_noalloc(&s, q, k, v, la, be, S0, NULL, o, ST, NULL),
           GDN_OK);
    gdn_shape huge = shape(1, 8192, 16, 128, 128, 64, 0, GDN_BF16, GDN_F32, 0);
    gdn_shape toolong = shape(1, 1 << 20, 64, 128, 128, 64, 0, GDN_BF16, GDN_F32, 0);
    expect("kda too long", gdn_kda_fwd_workspace_size(&toolong, &bytes), GDN_ERR_INVALID_ARG);
    if (!strstr(gdn_last_error(), "gdn_kda_fwd")) { printf("FAIL kda message\n"); ++failures; }
    expect("kda noalloc too large", gdn_kda_fwd_noalloc(&huge, q, k, v, la, be, NULL, NULL, o,
                                                        NULL, NULL), GDN_ERR_WORKSPACE);
    printf("noalloc max workspace %zu\n", gdn_kda_fwd_noalloc_max_workspace());

    /* Gated DeltaNet-2 */
    expect("gdn2 ws", gdn_gdn2_fwd_workspace_size(&s, &bytes), GDN_OK);
    expect("gdn2 misaligned ws", gdn_gdn2_fwd(&s, q, k, v, la, be, la, S0, NULL, o, ST, mis,
                                              bytes, NULL), GDN_ERR_ALIGNMENT);
    expect("gdn2 ok", gdn_gdn2_fwd(&s, q, k, v, la, be, la, S0, NULL, o, ST, ws, bytes, NULL),
           GDN_OK);

    /* decode step */
    expect("step bad dims", gdn_step(0, 4, 128, 128, GDN_BF16, GDN_F32, 0, q, k, v, la, be, ST,
                                     o, NULL), GDN_ERR_INVALID_ARG);
    expect("step alias", gdn_step(2, 4, 128, 128, GDN_BF16, GDN_F32, 0, q, k, v, la, be, ST,
                                  ST, NULL), GDN_ERR_INVALID_ARG);
    expect("step ok", gdn_step(2, 4, 128, 128, GDN_BF16, GDN_F32, 3, q, k, v, la, be, ST, o,
                               NULL), GDN_OK);
    printf("%d launches reached, %d failures\n", g_launches, failures);
    return failures != 0;
}
