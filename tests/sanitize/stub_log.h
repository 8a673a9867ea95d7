// The record of the last launch the stub launchers received.
#pragma once

#include "../../rwkv_linear_attention_amd/csrc/wkv7_launch.h"

struct StubLog {
    int calls = 0;
    char kind[16] = {0};
    int B = 0, T = 0, H = 0;
    long long n = 0;
    wkv7::SeqArgs seq{};
    wkv7::BwdArgs bwd{};
};
extern StubLog g_log;
