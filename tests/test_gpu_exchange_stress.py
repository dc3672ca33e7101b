"""Stress test of the tagged-word exchange (mk_selftest_exchange): the decode kernel's
own publish and gather code, run by the full persistent grid for many all-to-all
rounds, all to all (written through) and inside each XCD (plain stores, the local hops).  No word may be read with the right tag and a wrong value, no wait may give up
under the default spin limit, and a spin limit of one poll round must end every
workgroup's loop cleanly (the give-up path), with the timeout latched in the device
error word."""
import pytest

pytestmark = pytest.mark.gpu

DEV_ERR_TIMEOUT = 4


def test_exchange_stress_all_to_all():
    from persistent_megakernel_loop_amd.binding import selftest_exchange

    print("[case] exchange stress: 100000 all-to-all rounds of 256 x 64 words", flush=True)
    bad, gave_up, err, _ = selftest_exchange(100_000)
    print(f"[case] mismatched={bad} gave_up={gave_up} err={err}", flush=True)
    assert (bad, gave_up, err) == (0, 0, 0)


def test_exchange_stress_xcd_local_plain_stores():
    """The decode kernel's local hops: words stored plainly into the writer XCD's L2 and
    read there by device-coherent loads of the 31 other workgroups of that XCD."""
    from persistent_megakernel_loop_amd.binding import selftest_exchange

    print("[case] exchange stress: 200000 XCD-local rounds of 32 x 64 words, plain stores", flush=True)
    bad, gave_up, err, plain = selftest_exchange(200_000, xcd_local=True)
    print(f"[case] mismatched={bad} gave_up={gave_up} err={err} plain={plain}", flush=True)
    assert (bad, gave_up, err) == (0, 0, 0)
    assert plain == 1, "placement check failed: the workgroups did not sit on XCD b % 8"


def test_exchange_give_up_path():
    from persistent_megakernel_loop_amd.binding import selftest_exchange

    print("[case] exchange stress with a spin limit of one poll round", flush=True)
    bad, gave_up, err, _ = selftest_exchange(1000, spin_limit=1)
    print(f"[case] mismatched={bad} gave_up={gave_up} err={err}", flush=True)
    assert bad == 0 and gave_up > 0 and err & DEV_ERR_TIMEOUT
