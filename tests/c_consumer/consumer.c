/* A C11 program against include/qkvf.h and the built libqkvfront.so: the
 * header must compile as C and the exports must link from C.  It calls only
 * entries that answer without a GPU (launch shapes, status texts, refusals
 * decided before any device is touched).  Prints one line per failed
 * expectation, then "failures N", and exits with N. */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qkvf.h"

static int failures = 0;

static void expect(const char *what, long got, long want)
{
    if (got != want) {
        printf("FAIL %s: got %ld, want %ld\n", what, got, want);
        ++failures;
    }
}

int main(void)
{
    int grid = 0, splits = 0, waves = 0, tiles = 0;

    /* 8 KV heads: each XCD owns 18 whole heads, 4 K splits, 9 tiles a block. */
    expect("plan 9216/8", qkvf_plan(9216, 8, &grid, &splits, &waves, &tiles), QKVF_OK);
    expect("grid", grid, 256);
    expect("waves", waves, 8);
    expect("splits 9216/8", splits, 4);
    expect("tiles 9216/8", tiles, 9);
    /* 1 KV head: balanced rows, 8 K splits, a 4-row tile and two of 16. */
    expect("plan 1152/1", qkvf_plan(1152, 1, NULL, &splits, NULL, &tiles), QKVF_OK);
    expect("splits 1152/1", splits, 8);
    expect("tiles 1152/1", tiles, 3);
    /* 2 KV heads: 4 K splits below 12 token rows, 8 from 12 on. */
    expect("plan 2304/11", qkvf_plan(2304, 11, NULL, &splits, NULL, &tiles), QKVF_OK);
    expect("splits 2304/11", splits, 4);
    expect("tiles 2304/11", tiles, 3);
    expect("plan 2304/12", qkvf_plan(2304, 12, NULL, &splits, NULL, &tiles), QKVF_OK);
    expect("splits 2304/12", splits, 8);
    expect("tiles 2304/12", tiles, 5);
    expect("plan bad N", qkvf_plan(1000, 1, NULL, NULL, NULL, NULL), QKVF_ERR_SHAPE);
    expect("plan bad M", qkvf_plan(1152, 17, NULL, NULL, NULL, NULL), QKVF_ERR_ROWS);

    /* One request of 32K keys over 8 KV heads takes 32 split slots. */
    int z = 0;
    expect("attn2 plan", qkvf_attn2_plan(8, 32768, 0, 1, &z), QKVF_OK);
    expect("attn2 splits", z, 32);

    /* Refusals that come before any device call. */
    expect("prepare shape", qkvf_prepare(1000, 1, 1), QKVF_ERR_SHAPE);
    expect("prepare rows", qkvf_prepare(1152, 1, 0), QKVF_ERR_ROWS);
    expect("route tokens", qkvf_route(NULL, 256, NULL, 1.0, 0, NULL, NULL, NULL), QKVF_ERR_ROWS);
    expect("handoff mode", qkvf_set_handoff(2), QKVF_ERR_RANGE);
    expect("workspace", qkvf_workspace_bytes() > 0, 1);

    for (int s = QKVF_OK; s <= QKVF_ERR_TIMEOUT; ++s) {
        const char *text = qkvf_strerror(s);
        expect("strerror", text != NULL && strlen(text) > 0, 1);
    }
    expect("strerror unknown", qkvf_strerror(-1) != NULL, 1);

    printf("failures %d\n", failures);
    return failures;
}
